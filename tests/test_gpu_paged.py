"""Paged caches: indexer_score_paged(_rows) and hybrid_attn_decode_paged read a
query's keys / entries through a block table (硅星人 article, classic-cache
paragraph: fixed 128-token blocks of 32 CSA entries).  The same rows, paged
in shuffled blocks of a pool, must give the bits of the contiguous calls --
scores, selected sets and attention outputs -- for every block size."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, dev, gpu_bytes

pytestmark = pytest.mark.gpu


def _paginate(rows, n_ent, off, BR, rng, spare=3):
    """Pool of shuffled blocks holding each query's rows, and the block table.
    Unused pool rows hold random bytes; unused table entries name random
    blocks of the pool."""
    n_ent = np.asarray(n_ent, np.int64)
    nb = (n_ent + BR - 1) // BR
    bps = int(max(1, nb.max()))
    total = int(nb.sum()) + spare
    perm = rng.permutation(total).astype(np.int32)
    rb = rows.shape[1]
    pool = rng.integers(0, 256, size=(total * BR, rb), dtype=np.uint8)
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


def _indexer_pair(inp, BR, seed):
    B, ld = inp.B, int(max(1, inp.n_ent.max()))
    keys = inp.keys.reshape(-1, synth.row_bytes(inp.idx_fmt, inp.d_I))
    pool, table, bps, pool_rows = _paginate(keys, inp.n_ent, inp.kv_off, BR, np.random.default_rng(seed))
    q_idx, w, q_pos = dev(inp.q_idx), dev(inp.w), dev(inp.q_pos)
    a = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    b = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(q_idx, w, B, inp.H_I, inp.d_I, dev(inp.keys), inp.idx_fmt, dev(inp.kv_off), q_pos,
                      inp.m, a, ld)
    csa.indexer_score_paged(q_idx, w, B, inp.H_I, inp.d_I, dev(pool), inp.idx_fmt, pool_rows, dev(table), bps,
                            BR, q_pos, inp.m, b, ld)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("idx_fmt,H_I,BR", [(csa.FP8, 64, 32), (csa.FP8, 64, 16), (csa.FP8, 16, 256),
                                            (csa.FP8, 128, 64), (csa.MXFP4, 64, 32), (csa.MXFP4, 32, 128)])
def test_indexer_paged_matches_contiguous_bits(idx_fmt, H_I, BR):
    lengths = [65536, 9001, 2052, 130, 5, 3, 40000, 4096]
    inp = synth.decode_inputs(600 + BR + H_I, lengths, m=4, H=16, D=512, R=64, idx_fmt=idx_fmt, H_I=H_I)
    a, b = _indexer_pair(inp, BR, 7)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_indexer_paged_long_rows_interleaved_shares():
    """Rows long enough that the waves of a query take its groups in turn."""
    lengths = [262144, 262144, 100000, 262144, 50000, 262144, 8, 180000]
    inp = synth.decode_inputs(611, lengths, m=4, H=16, D=512, R=64, idx_fmt=csa.FP8, H_I=64)
    a, b = _indexer_pair(inp, 32, 8)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("H_I,BR,fmt", [(64, 32, csa.FP8), (32, 16, csa.FP8), (128, 64, csa.FP8),
                                        (64, 32, csa.MXFP4)])
def test_indexer_paged_rows_matches_contiguous_bits(H_I, BR, fmt):
    """A prefill chunk of two sequences (1,102 queries: FP8 takes the
    shared-key kernel, one workgroup's query block straddling the two sequences)
    reads each sequence's keys through one shared block-table row
    (q_block_row) of a table with spare rows; the scores carry the bits of
    indexer_score over the same keys stored contiguously.  So do the same
    queries with one table row each (q_block_row NULL), and a small batch of
    picked queries (the streaming kernel) naming the shared rows."""
    gen = synth.device_generator(81 + H_I + BR)
    rng = np.random.default_rng(82 + H_I + BR)
    m, d_I = 4, 128
    n_a, n_b = 40000, 5000
    keys = synth.device_rows(gen, n_a + n_b, d_I, fmt)
    nq_a, nq_b = 701, 401
    q_pos = np.concatenate([rng.integers(0, n_a * m, nq_a), rng.integers(0, n_b * m, nq_b)]).astype(np.int64)
    q_pos[:8] = [n_a * m - 1, 3, 64 * m - 1, 64 * m, 2048 * m + 5, n_a * m - 2, 0, 17]
    key_off = np.concatenate([np.zeros(nq_a), np.full(nq_b, n_a)]).astype(np.int64)
    nq = nq_a + nq_b
    q_idx = synth.device_rows(gen, nq * H_I, d_I, fmt).reshape(nq, H_I, -1)
    w = torch.rand((nq, H_I), generator=gen, device=DEV, dtype=torch.float32)
    ld = n_a
    ref = torch.full((nq, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(q_idx, w, nq, H_I, d_I, keys, fmt, dev(key_off), dev(q_pos), m, ref, ld)
    rb = synth.row_bytes(fmt, d_I)
    pool, tab2, bps, pool_rows = _paginate(keys.cpu().numpy().reshape(-1, rb), [n_a, n_b], [0, n_a], BR, rng)
    table = rng.integers(0, pool_rows // BR, size=(4, bps)).astype(np.int32)   # rows 0 and 2: spare
    table[1], table[3] = tab2[0], tab2[1]
    q_row = np.array([1] * nq_a + [3] * nq_b, np.int32)
    pool_d, q_pos_d = dev(pool), dev(q_pos)
    got = torch.full((nq, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score_paged_rows(q_idx, w, nq, H_I, d_I, pool_d, fmt, pool_rows, dev(table), 4, bps, BR,
                                 dev(q_row), q_pos_d, m, got, ld)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32)), "shared table rows: bits differ"
    if H_I == 64 and fmt == csa.FP8:
        per_q = torch.full((nq, ld), -7.0, dtype=torch.float32, device=DEV)
        csa.indexer_score_paged_rows(q_idx, w, nq, H_I, d_I, pool_d, fmt, pool_rows, dev(table[q_row]), nq, bps,
                                     BR, None, q_pos_d, m, per_q, ld)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int32), per_q.view(torch.int32)), "a table row per query: bits differ"
    # rows outside the table are clamped into it: A in row 0 and B in the
    # last row, named by -3 and 99 (the host check is bypassed)
    table_c = table[[1, 0, 2, 3]]
    q_row_c = np.array([-3] * nq_a + [99] * nq_b, np.int32)
    clamped = torch.full((nq, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score_paged_rows(q_idx, w, nq, H_I, d_I, pool_d, fmt, pool_rows, dev(table_c), 4, bps, BR,
                                 dev(q_row_c), q_pos_d, m, clamped, ld, check=False)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), clamped.view(torch.int32)), "clamped table rows: bits differ"
    picks = np.array([0, 1, 2, 4, 7, 350, 699, 700, 701, 702, 1100, 1101])
    pk = torch.as_tensor(picks, device=DEV)
    small = torch.full((len(picks), ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score_paged_rows(q_idx[pk].contiguous(), w[pk].contiguous(), len(picks), H_I, d_I, pool_d, fmt,
                                 pool_rows, dev(table), 4, bps, BR, dev(q_row[picks]), dev(q_pos[picks]), m, small,
                                 ld)
    torch.cuda.synchronize()
    assert torch.equal(ref[pk].view(torch.int32), small.view(torch.int32)), "picked queries: bits differ"


def _ring(win, win_len, rng):
    """The window rows of every query moved into a ring at a random start;
    the ring's other slots hold random bytes."""
    B, n_win, rb = win.shape
    ring = rng.integers(0, 256, size=win.shape, dtype=np.uint8)
    start = rng.integers(0, n_win, size=B).astype(np.int32)
    for b in range(B):
        for t in range(int(win_len[b])):
            ring[b, (start[b] + t) % n_win] = win[b, t]
    return ring, start


def _attn_pair(inp, sel, BR, seed, variant, ring=False, hca=False):
    B, H, D = inp.B, inp.H, inp.D
    rb = synth.row_bytes(csa.SPLIT, D, inp.R)
    rng = np.random.default_rng(seed)
    pool, table, bps, pool_rows = _paginate(inp.kv.reshape(-1, rb), inp.n_ent, inp.kv_off, BR, rng)
    q, q_pos, win, win_len, sinks = dev(inp.q), dev(inp.q_pos), dev(inp.win), dev(inp.win_len), dev(inp.sinks)
    pwin, pstart = win, None
    if ring:
        r, st = _ring(inp.win, inp.win_len, rng)
        pwin, pstart = dev(r), dev(st)
    idx = None if hca else dev(sel)
    k = 0 if hca else inp.k
    outs = []
    for paged in (False, True):
        out = gpu_bytes(B * H * D * 2)
        if paged:
            csa.hybrid_attn_decode_paged(q, csa.BF16, B, H, D, q_pos, None, EPS, inp.R, ROPE_BASE, dev(pool),
                                         csa.SPLIT, pool_rows, dev(table), bps, BR, inp.m, idx, k, pwin,
                                         csa.BF16, inp.n_win, win_len, sinks, inp.scale, out, csa.BF16, variant,
                                         win_start=pstart)
        else:
            csa.hybrid_attn_decode(q, csa.BF16, B, H, D, q_pos, None, EPS, inp.R, ROPE_BASE, dev(inp.kv),
                                   csa.SPLIT, dev(inp.kv_off), inp.m, idx, k, win, csa.BF16, inp.n_win,
                                   win_len, sinks, inp.scale, out, csa.BF16, variant)
        outs.append(out)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("BR,k,variant", [(32, 512, csa.VARIANT_AUTO), (1, 512, csa.VARIANT_LOW_OCC),
                                          (128, 1024, csa.VARIANT_HIGH_OCC), (32, 64, csa.VARIANT_AUTO),
                                          (32, 2048, csa.VARIANT_AUTO), (32, 512, csa.VARIANT_FULL_DIMS)])
def test_attention_paged_matches_contiguous_bits(BR, k, variant):
    lengths = [65536, 9001, 2052, 130, 5, 3, 40000]
    inp = synth.decode_inputs(620 + BR, lengths, m=4, H=64, D=512, R=64, k=k)
    sel = synth.random_selection(np.random.default_rng(9), inp.n_ent, k)
    a, b = _attn_pair(inp, sel, BR, 10, variant)
    assert torch.equal(a, b)


@pytest.mark.parametrize("BR,variant", [(1, csa.VARIANT_AUTO), (4, csa.VARIANT_LOW_OCC), (16, csa.VARIANT_AUTO),
                                        (2, csa.VARIANT_FULL_DIMS)])
def test_hca_attention_paged_matches_contiguous_bits(BR, variant):
    """HCA (every visible entry attended; one entry per 128-token block at
    block_rows = 1), with lists past 1024 positions mapped inside the loop."""
    lengths = [262144, 40000, 128, 127, 9000, 300000]
    inp = synth.decode_inputs(660 + BR, lengths, m=128, H=64, D=512, R=64, csa=False)
    a, b = _attn_pair(inp, None, BR, 15, variant, ring=True, hca=True)
    assert torch.equal(a, b)


@pytest.mark.parametrize("variant", [csa.VARIANT_AUTO, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS])
def test_attention_window_ring_matches_rows_in_order(variant):
    """The request's window kept as a ring (random start, random bytes in the
    free slots) gives the bits of the window stored in order."""
    lengths = [65536, 9001, 2052, 130, 5, 3, 40000, 100]
    inp = synth.decode_inputs(650, lengths, m=4, H=64, D=512, R=64, k=512)
    sel = synth.random_selection(np.random.default_rng(13), inp.n_ent, 512)
    a, b = _attn_pair(inp, sel, 32, 14, variant, ring=True)
    assert torch.equal(a, b)


def test_paged_step_matches_contiguous_step():
    """indexer -> top-k -> attention over paged caches (blocks of 32 entries:
    one 128-token block of CSA entries) against the same step on contiguous
    caches: the same selected sets and output bits."""
    lengths = [65536, 20000, 4100, 129, 70000, 3]
    inp = synth.decode_inputs(631, lengths, m=4, H=64, D=512, R=64, k=512)
    B, ld, k = inp.B, int(inp.n_ent.max()), inp.k
    a, b = _indexer_pair(inp, 32, 11)
    nv = dev(inp.n_ent)
    ia = torch.empty((B, k), dtype=torch.int32, device=DEV)
    ib = torch.empty((B, k), dtype=torch.int32, device=DEV)
    csa.topk_select(a, ld, B, nv, k, ia)
    csa.topk_select(b, ld, B, nv, k, ib)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib)
    oa, ob = _attn_pair(inp, ia.cpu().numpy(), 32, 12, csa.VARIANT_AUTO)
    assert torch.equal(oa, ob)


def test_paged_argument_errors():
    inp = synth.decode_inputs(640, [4096, 2052], m=4, H=16, D=512, R=64, H_I=64)
    B, ld = inp.B, int(inp.n_ent.max())
    keys = dev(inp.keys)
    table = torch.zeros((B, 200), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, ld), dtype=torch.float32, device=DEV)
    args = (dev(inp.q_idx), dev(inp.w), B, 64, 128, keys, csa.FP8, int(inp.n_ent.sum()), table, 200)
    with pytest.raises(csa.CsaError):                       # block_rows not a power of two
        csa.indexer_score_paged(*args, 24, dev(inp.q_pos), 4, scores, ld, check=False)
    with pytest.raises(csa.CsaError):                       # below 16 rows per block
        csa.indexer_score_paged(*args, 8, dev(inp.q_pos), 4, scores, ld, check=False)
    with pytest.raises(ValueError):                         # a query sees more rows than its table row holds
        csa.indexer_score_paged(dev(inp.q_idx), dev(inp.w), B, 64, 128, keys, csa.FP8, int(inp.n_ent.sum()),
                                table[:, :1].contiguous(), 1, 16, dev(inp.q_pos), 4, scores, ld)


def test_one_block_table_serves_the_csa_and_hca_pools():
    """The classic cache's 128-token block (硅星人 article, classic-cache
    paragraph): token block j of a sequence holds its 32 CSA entries (m = 4)
    and its one HCA entry (m' = 128).  One block table per sequence names the
    block in both pools -- CSA rows at block_rows = 32, HCA rows at
    block_rows = 1 -- and the paged CSA and HCA attentions give the
    contiguous calls' bits through it."""
    lengths = [65636, 9000, 300, 640, 127]
    ci = synth.decode_inputs(701, lengths, m=4, H=64, D=512, R=64, k=512)
    hi = synth.decode_inputs(702, lengths, m=128, H=64, D=512, R=64, csa=False)
    rb = synth.row_bytes(csa.SPLIT, 512, 64)
    rng = np.random.default_rng(703)
    nb = (ci.n_ent.astype(np.int64) + 31) // 32                 # token blocks (of 128) per sequence
    assert np.all(hi.n_ent <= nb)
    total = int(nb.sum()) + 2
    bps = int(max(1, nb.max()))
    perm = rng.permutation(total).astype(np.int32)
    table = rng.integers(0, total, size=(len(lengths), bps)).astype(np.int32)
    csa_pool = rng.integers(0, 256, size=(total * 32, rb), dtype=np.uint8)
    hca_pool = rng.integers(0, 256, size=(total, rb), dtype=np.uint8)
    crow, hrow = ci.kv.reshape(-1, rb), hi.kv.reshape(-1, rb)
    nxt = 0
    for i in range(len(lengths)):
        for j in range(int(nb[i])):
            blk = int(perm[nxt])
            nxt += 1
            table[i, j] = blk
            lo, cnt = int(ci.kv_off[i]) + 32 * j, min(32, int(ci.n_ent[i]) - 32 * j)
            csa_pool[blk * 32: blk * 32 + cnt] = crow[lo: lo + cnt]
            if j < int(hi.n_ent[i]):
                hca_pool[blk] = hrow[int(hi.kv_off[i]) + j]
    sel = synth.random_selection(np.random.default_rng(704), ci.n_ent, ci.k)
    tab = dev(table)
    for inp, pool, BR, idx, k in ((ci, csa_pool, 32, dev(sel), ci.k), (hi, hca_pool, 1, None, 0)):
        B, H, D = inp.B, inp.H, inp.D
        q, q_pos, win, win_len, sinks = dev(inp.q), dev(inp.q_pos), dev(inp.win), dev(inp.win_len), dev(inp.sinks)
        a, b = gpu_bytes(B * H * D * 2), gpu_bytes(B * H * D * 2)
        csa.hybrid_attn_decode(q, csa.BF16, B, H, D, q_pos, None, EPS, inp.R, ROPE_BASE, dev(inp.kv), csa.SPLIT,
                               dev(inp.kv_off), inp.m, idx, k, win, csa.BF16, inp.n_win, win_len, sinks, inp.scale,
                               a, csa.BF16, csa.VARIANT_AUTO)
        csa.hybrid_attn_decode_paged(q, csa.BF16, B, H, D, q_pos, None, EPS, inp.R, ROPE_BASE, dev(pool), csa.SPLIT,
                                     pool.shape[0], tab, bps, BR, inp.m, idx, k, win, csa.BF16, inp.n_win, win_len,
                                     sinks, inp.scale, b, csa.BF16, csa.VARIANT_AUTO)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"m = {inp.m}: paged output differs"

"""Causal prefill on the GPU: a chunk of new query tokens after a cached
context, each with its own selected entries and its own 128-token window
(DeepSeek-V4 blog, index visibility: every query sees floor((p+1)/m) entries;
Partial RoPE paragraph: the window of raw tokens).  Checked against the
oracle on sampled queries, across variants, and against decode: a token gets
the same bits from prefill as from decode given the same entries and window
rows (QbitAI piece on batch invariance)."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, assert_lowp_close, dev, gpu_bytes
from oracle import formats as OF
from oracle import method as OM

pytestmark = pytest.mark.gpu

D, R, N_WIN = 512, 64, 128


def _case(seed, cached, chunk, H, m, k):
    rng = synth.rng_for(seed)
    T = cached + chunk
    kv = synth.random_rows(rng, T // m, D, csa.SPLIT, R)
    tok_pos0 = max(0, cached - N_WIN + 1)
    tok = synth.random_rows(rng, T - tok_pos0, D, csa.BF16)
    q = synth.random_rows(rng, chunk * H, D, csa.BF16).reshape(chunk, H, -1)
    q_pos = (cached + np.arange(chunk)).astype(np.int64)
    n_ent = (q_pos + 1) // m
    sel = synth.random_selection(rng, n_ent, k) if k else None
    sinks = rng.standard_normal(H).astype(np.float32)
    return dict(kv=kv, tok=tok, tok_pos0=tok_pos0, q=q, q_pos=q_pos, n_ent=n_ent, sel=sel,
                sinks=sinks, H=H, m=m, k=k, chunk=chunk, scale=1.0 / np.sqrt(D))


def _prefill(c, variant, bufs=None):
    nq, H = c["chunk"], c["H"]
    if bufs is None:
        bufs = dict(q=dev(c["q"]), q_pos=dev(c["q_pos"]), kv=dev(c["kv"]),
                    kv_off=torch.zeros(nq, dtype=torch.int64, device=DEV), tok=dev(c["tok"]),
                    tok_off=torch.zeros(nq, dtype=torch.int64, device=DEV),
                    tok_pos0=torch.full((nq,), c["tok_pos0"], dtype=torch.int64, device=DEV),
                    sinks=dev(c["sinks"]), idx=dev(c["sel"]) if c["sel"] is not None else None)
    out = gpu_bytes(nq * H * 2 * D)
    csa.hybrid_attn_prefill(bufs["q"], csa.BF16, nq, H, D, bufs["q_pos"], None, EPS, R, ROPE_BASE,
                            bufs["kv"], csa.SPLIT, bufs["kv_off"], c["m"], bufs["idx"], c["k"],
                            bufs["tok"], csa.BF16, bufs["tok_off"], bufs["tok_pos0"], N_WIN,
                            bufs["sinks"], c["scale"], out, csa.BF16, variant)
    return out.view(nq, H * 2 * D).cpu().numpy(), bufs


@pytest.mark.parametrize("cached,chunk,H,m,k", [
    (4096, 96, 64, 4, 256),        # CSA: selected entries + window
    (2048, 80, 32, 128, 0),        # HCA: every entry + window
    (60, 70, 16, 4, 64),           # short context: windows cut at position 0
])
def test_prefill_matches_oracle(cached, chunk, H, m, k):
    c = _case(11 + cached, cached, chunk, H, m, k)
    got, _ = _prefill(c, csa.VARIANT_AUTO)
    ents_all = OF.decode_rows(c["kv"], csa.SPLIT, D, R)
    tok_rows = OF.decode_rows(c["tok"], csa.BF16, D)
    q = OF.decode_rows(c["q"].reshape(chunk * H, -1), csa.BF16, D).reshape(chunk, H, D)
    for i in sorted({0, 1, chunk // 2, chunk - 1, 7 % chunk}):
        N = int(c["n_ent"][i])
        sel = c["sel"][i][c["sel"][i] >= 0] if c["sel"] is not None else None
        ref = OM.prefill_one(q[i], int(c["q_pos"][i]), ents_all[:N], tok_rows, c["tok_pos0"],
                             c["sinks"].astype(np.float64), c["scale"], m, N_WIN, idx=sel,
                             eps=EPS, R=R, base=ROPE_BASE)
        g = OF.decode_rows(got[i].reshape(H, -1), csa.BF16, D)
        assert_lowp_close(g, ref, what=f"prefill query {i}")


def test_prefill_bits_match_decode_and_variants():
    c = _case(5, 3000, 64, 64, 4, 512)
    nq, H = c["chunk"], c["H"]
    base, bufs = _prefill(c, csa.VARIANT_AUTO)
    for v in (csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS):
        got, _ = _prefill(c, v, bufs)
        assert np.array_equal(got, base), f"variant {v} changed the bits"
    # decode of the same tokens, with their window rows copied out of the run
    rb = 2 * D
    for i in (0, 17, nq - 1):
        p = int(c["q_pos"][i])
        first = max(0, p - N_WIN + 1, c["tok_pos0"])
        rows = c["tok"][first - c["tok_pos0"]: p - c["tok_pos0"] + 1]
        win = np.zeros((1, N_WIN, rb), np.uint8)
        win[0, : rows.shape[0]] = rows
        out = gpu_bytes(H * rb)
        csa.hybrid_attn_decode(bufs["q"][i:i + 1].contiguous(), csa.BF16, 1, H, D,
                               bufs["q_pos"][i:i + 1].contiguous(), None, EPS, R, ROPE_BASE,
                               bufs["kv"], csa.SPLIT, bufs["kv_off"][:1].contiguous(), c["m"],
                               bufs["idx"][i:i + 1].contiguous(), c["k"], dev(win), csa.BF16, N_WIN,
                               torch.tensor([rows.shape[0]], dtype=torch.int32, device=DEV),
                               bufs["sinks"], c["scale"], out, csa.BF16)
        assert np.array_equal(out.cpu().numpy(), base[i]), f"query {i}: decode bits differ from prefill"


def _paginate_one(rows, BR, rng, total_spare=3):
    """One sequence's rows in shuffled blocks of a pool; unused pool rows and
    unused table entries hold random values."""
    n = rows.shape[0]
    nb = max(1, (n + BR - 1) // BR)
    total = nb + total_spare
    perm = rng.permutation(total).astype(np.int32)[:nb]
    pool = rng.integers(0, 256, size=(total * BR, rows.shape[1]), dtype=np.uint8)
    for j in range(nb):
        cnt = min(BR, n - j * BR)
        if cnt > 0:
            pool[perm[j] * BR: perm[j] * BR + cnt] = rows[j * BR: j * BR + cnt]
    return pool, perm, total * BR


@pytest.mark.parametrize("m,k,BR", [(4, 256, 32), (4, 512, 1), (128, 0, 1), (128, 0, 4)])
def test_prefill_paged_matches_contiguous_bits(m, k, BR):
    """Two sequences in one chunk (classic cache of the 硅星人 article): each
    sequence's entries in shuffled blocks of one shared pool; its queries all
    read the sequence's block-table row (q_block_row), and the table holds
    spare rows that no query reads.  The bits equal hybrid_attn_prefill over
    the same entries stored contiguously, per query and for every variant;
    without q_block_row (one table row per query) they are the same again."""
    rng = np.random.default_rng(4100 + m + k + BR)
    H = 32
    a = _case(700 + m + BR, 3000 if m == 4 else 20000, 48, H, m, k)
    b = _case(900 + m + BR, 500 if m == 4 else 1100, 40, H, m, k)
    rb, tb = synth.row_bytes(csa.SPLIT, D, R), 2 * D
    na, nb = a["chunk"], b["chunk"]
    nq = na + nb
    # contiguous: a's entries then b's; a's token rows then b's
    kv = np.concatenate([a["kv"], b["kv"]])
    tok = np.concatenate([a["tok"], b["tok"]])
    kv_off = np.array([0] * na + [a["kv"].shape[0]] * nb, np.int64)
    tok_off = np.array([0] * na + [a["tok"].shape[0]] * nb, np.int64)
    tok_pos0 = np.array([a["tok_pos0"]] * na + [b["tok_pos0"]] * nb, np.int64)
    q = np.concatenate([a["q"], b["q"]])
    q_pos = np.concatenate([a["q_pos"], b["q_pos"]])
    sel = np.concatenate([a["sel"], b["sel"]]) if k else None
    sinks, scale = a["sinks"], a["scale"]
    # paged: both sequences' blocks in one pool, table rows [spare, a, spare, b]
    pa, perm_a, rows_a = _paginate_one(a["kv"], BR, rng)
    pb, perm_b, rows_b = _paginate_one(b["kv"], BR, rng)
    pool = np.concatenate([pa, pb])
    blk_a = perm_a
    blk_b = perm_b + rows_a // BR
    bps = max(len(blk_a), len(blk_b)) + 2
    total_blocks = pool.shape[0] // BR
    table = rng.integers(0, total_blocks, size=(4, bps)).astype(np.int32)
    table[1, : len(blk_a)] = blk_a
    table[3, : len(blk_b)] = blk_b
    q_row = np.array([1] * na + [3] * nb, np.int32)
    g = dict(q=dev(q), q_pos=dev(q_pos), kv=dev(kv), kv_off=dev(kv_off), tok=dev(tok), tok_off=dev(tok_off),
             tok_pos0=dev(tok_pos0), sinks=dev(sinks), idx=dev(sel) if k else None)
    pool_d, table_d, q_row_d = dev(pool), dev(table), dev(q_row)
    per_q = dev(table[q_row])                            # one table row per query
    table_c = dev(table[[1, 0, 2, 3]])
    q_row_c = dev(np.array([-3] * na + [99] * nb, np.int32))
    for v in (csa.VARIANT_AUTO, csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS):
        ref = gpu_bytes(nq * H * tb)
        csa.hybrid_attn_prefill(g["q"], csa.BF16, nq, H, D, g["q_pos"], None, EPS, R, ROPE_BASE, g["kv"], csa.SPLIT,
                                g["kv_off"], m, g["idx"], k, g["tok"], csa.BF16, g["tok_off"], g["tok_pos0"], N_WIN,
                                g["sinks"], scale, ref, csa.BF16, v)
        got = gpu_bytes(nq * H * tb)
        csa.hybrid_attn_prefill_paged(g["q"], csa.BF16, nq, H, D, g["q_pos"], None, EPS, R, ROPE_BASE, pool_d,
                                      csa.SPLIT, pool.shape[0], table_d, 4, bps, BR, q_row_d, m, g["idx"], k,
                                      g["tok"], csa.BF16, g["tok_off"], g["tok_pos0"], N_WIN, g["sinks"], scale,
                                      got, csa.BF16, v)
        got2 = gpu_bytes(nq * H * tb)
        csa.hybrid_attn_prefill_paged(g["q"], csa.BF16, nq, H, D, g["q_pos"], None, EPS, R, ROPE_BASE, pool_d,
                                      csa.SPLIT, pool.shape[0], per_q, nq, bps, BR, None, m, g["idx"], k,
                                      g["tok"], csa.BF16, g["tok_off"], g["tok_pos0"], N_WIN, g["sinks"], scale,
                                      got2, csa.BF16, v)
        # rows outside the table clamp into it: A's row first, B's last (host check bypassed)
        got3 = gpu_bytes(nq * H * tb)
        csa.hybrid_attn_prefill_paged(g["q"], csa.BF16, nq, H, D, g["q_pos"], None, EPS, R, ROPE_BASE, pool_d,
                                      csa.SPLIT, pool.shape[0], table_c, 4, bps, BR, q_row_c, m, g["idx"], k,
                                      g["tok"], csa.BF16, g["tok_off"], g["tok_pos0"], N_WIN, g["sinks"], scale,
                                      got3, csa.BF16, v, check=False)
        torch.cuda.synchronize()
        assert torch.equal(ref, got3), f"variant {v}: clamped table rows differ"
        assert torch.equal(ref, got), f"variant {v}: paged prefill (shared table rows) differs from contiguous"
        assert torch.equal(ref, got2), f"variant {v}: paged prefill (a table row per query) differs"
    # the first query of each sequence against the oracle, from the pool through the table
    ents = OF.decode_rows(pool, csa.SPLIT, D, R)
    toks = OF.decode_rows(tok, csa.BF16, D)
    qf = OF.decode_rows(q.reshape(nq * H, -1), csa.BF16, D).reshape(nq, H, D)
    out = OF.decode_rows(ref.view(torch.uint8).cpu().numpy().reshape(nq * H, tb), csa.BF16, D).reshape(nq, H, D)
    for i in (0, na + nb - 1):
        c = a if i < na else b
        N = int((q_pos[i] + 1) // m)
        tr = table[q_row[i]]
        phys = [int(tr[e // BR]) * BR + e % BR for e in range(N)]
        s = sel[i][sel[i] >= 0] if k else None
        ref_i = OM.prefill_one(qf[i], int(q_pos[i]), ents[phys], toks[tok_off[i]:], int(tok_pos0[i]),
                               sinks.astype(np.float64), scale, m, N_WIN, idx=s, eps=EPS, R=R, base=ROPE_BASE)
        assert_lowp_close(out[i], ref_i, what=f"paged prefill query {i} ({'first' if c is a else 'second'} sequence)")

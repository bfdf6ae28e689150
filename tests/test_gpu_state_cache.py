"""A decode stream through the per-request state cache (硅星人 article, the
state-cache and classic-cache paragraphs): tokens arrive one per step; the
tokens of a block not yet complete wait in the caller's state, and the step
that completes a block compresses it into the next entry of a paged cache
(pool rows through a block table); every token's window row goes into a ring
of n_win slots.  After the stream the pool, read in logical order, holds the
bytes of one bulk csa_compress of every complete block; the ring holds the
bulk window rows of the last n_win tokens; and the last token's attention
over the paged cache and the ring equals the contiguous call bit for bit and
the oracle within the low-precision bar.  A stream saved to the host
mid-way, restored into fresh buffers and continued ends with the same bytes
and the same attention bits."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from oracle import formats as OF
from oracle import method as OM

from gpu_common import DEV, EPS, ROPE_BASE, assert_lowp_close, decode_out, dev, gpu_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


def _i64(v):
    return torch.as_tensor(np.asarray(v, np.int64), device=DEV)


def _compress(x, gate, n_tok, m, pos0, row, out, fmt, D, R):
    csa.csa_compress(x, csa.BF16, gate, 1, n_tok, D, m, 1, _i64([0, n_tok]), _i64([pos0]), _i64([row]),
                     1, None, EPS, R, ROPE_BASE, out, fmt)


@pytest.mark.parametrize("m,T,BR", [(4, 4 * 97 + 3, 32), (128, 128 * 3 + 5, 1)])
def test_state_cache_stream(m, T, BR):
    D, R, H, n_win = 512, 64, 16, 128
    rng = np.random.default_rng(900 + m)
    x = torch.as_tensor(rng.standard_normal((T, D), dtype=np.float32), device=DEV).to(torch.bfloat16)
    gate = torch.as_tensor(rng.standard_normal((T, 1), dtype=np.float32), device=DEV)
    rb = synth.row_bytes(csa.SPLIT, D, R)
    wb = synth.row_bytes(csa.BF16, D, R)
    n_ent = T // m
    # the classic cache: a pool of blocks of BR entries in a seeded order, with spare blocks
    n_blk = (n_ent + BR - 1) // BR
    total = n_blk + 3
    table = rng.permutation(total)[:n_blk].astype(np.int32)
    pool = torch.as_tensor(rng.integers(0, 256, size=(total * BR, rb), dtype=np.uint8), device=DEV)
    ring = torch.as_tensor(rng.integers(0, 256, size=(n_win, wb), dtype=np.uint8), device=DEV)
    phys = lambda j: int(table[j // BR]) * BR + j % BR  # noqa: E731
    # ---- the stream: one token per step
    for t in range(T):
        if (t + 1) % m == 0:                          # this token completes block j
            j = t // m
            _compress(x[t + 1 - m: t + 1], gate[t + 1 - m: t + 1], m, m, t + 1 - m, phys(j), pool, csa.SPLIT,
                      D, R)
        _compress(x[t: t + 1], gate[t: t + 1], 1, 1, t, t % n_win, ring, csa.BF16, D, R)
    # ---- the same tokens in bulk
    bulk = gpu_bytes(max(1, n_ent) * rb)
    _compress(x[: n_ent * m], gate[: n_ent * m], n_ent * m, m, 0, 0, bulk, csa.SPLIT, D, R)
    win_all = gpu_bytes(T * wb)
    _compress(x, gate, T, 1, 0, 0, win_all, csa.BF16, D, R)
    torch.cuda.synchronize()
    pool_h = pool.cpu().numpy()
    bulk_h = bulk.cpu().numpy().reshape(-1, rb)
    for j in range(n_ent):
        assert np.array_equal(pool_h[phys(j)], bulk_h[j]), f"entry {j}"
    ring_h = ring.cpu().numpy()
    win_h = win_all.cpu().numpy().reshape(T, wb)
    for s in range(n_win):
        t = T - 1 - ((T - 1 - s) % n_win)              # the newest token kept in slot s
        assert np.array_equal(ring_h[s], win_h[t]), f"ring slot {s}"
    # ---- the last token attends to every entry and its window: paged vs contiguous vs oracle
    p = T - 1
    q = rng.standard_normal((1, H, D), dtype=np.float32)
    q_b = torch.as_tensor(q, device=DEV).to(torch.bfloat16)
    sinks = rng.standard_normal(H).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    wl = min(n_win, p + 1)
    start = (p + 1 - wl) % n_win                      # ring slot of the oldest window row
    win_rows = win_all.view(torch.uint8).reshape(T, wb)[p + 1 - wl: p + 1].contiguous()
    out_c = gpu_bytes(H * D * 2)
    csa.hybrid_attn_decode(q_b, csa.BF16, 1, H, D, _i64([p]), None, EPS, R, ROPE_BASE, bulk, csa.SPLIT, _i64([0]),
                           m, None, 0, win_rows, csa.BF16, n_win, dev(np.array([wl], np.int32)), dev(sinks), scale,
                           out_c, csa.BF16, csa.VARIANT_AUTO)
    out_p = gpu_bytes(H * D * 2)
    csa.hybrid_attn_decode_paged(q_b, csa.BF16, 1, H, D, _i64([p]), None, EPS, R, ROPE_BASE, pool, csa.SPLIT,
                                 total * BR, dev(table), n_blk, BR, m, None, 0, ring, csa.BF16, n_win,
                                 dev(np.array([wl], np.int32)), dev(sinks), scale, out_p, csa.BF16,
                                 win_start=dev(np.array([start], np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p), "paged cache + ring differ from the contiguous call"
    ents = OF.decode_rows(bulk_h[:n_ent], csa.SPLIT, D, R)
    win = OF.decode_rows(win_h[p + 1 - wl: p + 1], csa.BF16, D, R)
    qh = OF.decode_rows(q_b.view(torch.uint8).cpu().numpy().reshape(H, 2 * D), csa.BF16, D, R)
    ref = OM.decode_one(qh, p, ents, win, sinks.astype(np.float64), scale, m, idx=None, eps=EPS, R=R,
                        base=ROPE_BASE)
    assert_lowp_close(decode_out(out_c, csa.BF16, 1, H, D)[0], ref, what=f"state-cache stream m={m}")


def _run_stream(x, gate, m, D, R, n_win, pool, ring, phys, t0, t1):
    for t in range(t0, t1):
        if (t + 1) % m == 0:
            j = t // m
            _compress(x[t + 1 - m: t + 1], gate[t + 1 - m: t + 1], m, m, t + 1 - m, phys(j), pool, csa.SPLIT, D, R)
        _compress(x[t: t + 1], gate[t: t + 1], 1, 1, t, t % n_win, ring, csa.BF16, D, R)


@pytest.mark.parametrize("m,T,BR,cut", [(4, 4 * 61 + 2, 16, 4 * 30 + 1), (128, 128 * 2 + 9, 1, 200)])
def test_cache_save_restore_continue(m, T, BR, cut):
    """Resume: the caches are the caller's memory, so saving them is a copy.
    A stream stopped after token `cut`, its paged pool and window ring copied
    to the host, restored into fresh buffers that held other bytes, and
    continued, ends with the bytes of the uninterrupted stream, and the last
    token's paged attention has the same bits."""
    D, R, H, n_win = 512, 64, 16, 128
    rng = np.random.default_rng(1000 + m)
    x = torch.as_tensor(rng.standard_normal((T, D), dtype=np.float32), device=DEV).to(torch.bfloat16)
    gate = torch.as_tensor(rng.standard_normal((T, 1), dtype=np.float32), device=DEV)
    rb, wb = synth.row_bytes(csa.SPLIT, D, R), synth.row_bytes(csa.BF16, D, R)
    n_blk = (T // m + BR - 1) // BR
    total = n_blk + 2
    table = rng.permutation(total)[:n_blk].astype(np.int32)
    phys = lambda j: int(table[j // BR]) * BR + j % BR  # noqa: E731
    fresh = lambda n, w: torch.as_tensor(rng.integers(0, 256, size=(n, w), dtype=np.uint8), device=DEV)  # noqa: E731
    pool_a, ring_a = fresh(total * BR, rb), fresh(n_win, wb)
    pool_b, ring_b = fresh(total * BR, rb), fresh(n_win, wb)
    pool_b.copy_(pool_a)
    ring_b.copy_(ring_a)
    # run A: uninterrupted
    _run_stream(x, gate, m, D, R, n_win, pool_a, ring_a, phys, 0, T)
    # run B: stop at `cut`, save to the host, restore into new buffers, continue
    _run_stream(x, gate, m, D, R, n_win, pool_b, ring_b, phys, 0, cut)
    torch.cuda.synchronize()
    saved_pool, saved_ring = pool_b.cpu(), ring_b.cpu()
    pool_c, ring_c = fresh(total * BR, rb), fresh(n_win, wb)
    pool_c.copy_(saved_pool.to(DEV))
    ring_c.copy_(saved_ring.to(DEV))
    del pool_b, ring_b
    _run_stream(x, gate, m, D, R, n_win, pool_c, ring_c, phys, cut, T)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_c), "the resumed pool differs"
    assert torch.equal(ring_a, ring_c), "the resumed window ring differs"
    p = T - 1
    q_b = torch.as_tensor(rng.standard_normal((1, H, D), dtype=np.float32), device=DEV).to(torch.bfloat16)
    sinks = dev(rng.standard_normal(H).astype(np.float32))
    wl = min(n_win, p + 1)
    start = dev(np.array([(p + 1 - wl) % n_win], np.int32))
    outs = []
    for pool, ring in ((pool_a, ring_a), (pool_c, ring_c)):
        out = gpu_bytes(H * D * 2)
        csa.hybrid_attn_decode_paged(q_b, csa.BF16, 1, H, D, _i64([p]), None, EPS, R, ROPE_BASE, pool, csa.SPLIT,
                                     total * BR, dev(table), n_blk, BR, m, None, 0, ring, csa.BF16, n_win,
                                     dev(np.array([wl], np.int32)), sinks, 1.0 / np.sqrt(D), out, csa.BF16,
                                     win_start=start)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "attention after the resume differs"

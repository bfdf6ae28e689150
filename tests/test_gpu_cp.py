"""Context-parallel compression of one long sequence, on one GPU (DeepSeek-V4
blog, 百万 token 怎么切分到多张卡): the sequence is cut into shards at token
boundaries that need not fall on blocks; each shard receives the last m
uncompressed tokens of the shard before it (a device copy stands in for the
send to the next rank), compresses them with its own tokens into a
fixed-length run of blocks (padding after its valid rows), the runs are
gathered into one buffer (the all-gather), and csa_select_and_pad joins them
with every padding row at the end.  The joined run must equal the compression
of the unsharded sequence byte for byte, and the oracle's entries within the
compressor's bar."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, dev
from test_gpu_parity import _compress_error_bound, _quant_ok
from oracle import formats as OF
from oracle import method as OM

pytestmark = pytest.mark.gpu


def _compress(x, gate, n_tok, D, m, pos0, row0, normalize, R, out, fmt):
    one = lambda v: dev(np.array(v, np.int64))  # noqa: E731
    csa.csa_compress(x, csa.BF16, gate, 1, n_tok, D, m, 1, one([0, n_tok]), one([pos0]), one([row0]), normalize,
                     None, EPS, R, ROPE_BASE, out, fmt)


def _cp_case(L, cuts, m, D, R, fmt, seed):
    normalize = R > 0
    rb = csa.row_bytes(fmt, D, R)
    tok = synth.token_inputs(seed, L, D)
    x = torch.from_numpy(tok.x).to(DEV).to(torch.bfloat16)
    g = dev(tok.gate)
    n_all = L // m
    # the unsharded sequence: one segment, blocks at 0, m, 2m, ...
    whole = torch.zeros(max(1, n_all) * rb, dtype=torch.uint8, device=DEV)
    if n_all:
        _compress(x[: n_all * m], g[: n_all * m], n_all * m, D, m, 0, 0, normalize, R, whole, fmt)
    # shards [b_s, b_s+1); every shard holds at least m tokens, so the
    # unfinished block it hands on lies inside its last m tokens
    b = [0] + list(cuts) + [L]
    S = len(b) - 1
    assert all(b[s + 1] - b[s] >= m for s in range(S))
    first = [(b[s] // m) * m for s in range(S)]               # first token of the shard's first block
    last = [(b[s + 1] // m) * m if s + 1 < S else n_all * m for s in range(S)]
    n_valid = [(last[s] - first[s]) // m for s in range(S)]
    cap = max(n_valid) + 1                                     # fixed run length, a little padding
    rng = np.random.default_rng(seed + 1)
    runs = dev(rng.integers(0, 256, size=(S * cap * rb,), dtype=np.uint8))   # padding rows hold anything
    for s in range(S):
        local = x[b[s]: b[s + 1]]
        lg = g[b[s]: b[s + 1]]
        if s > 0:                                              # the last m tokens of shard s - 1
            carry, cg = x[b[s] - m: b[s]].clone(), g[b[s] - m: b[s]].clone()
            buf, gb = torch.cat([carry, local]), torch.cat([cg, lg])
            start = m - (b[s] - first[s])                      # the carried tokens of the unfinished block
        else:
            buf, gb, start = local, lg, 0
        n_tok = n_valid[s] * m
        if n_tok:
            _compress(buf[start: start + n_tok].contiguous(), gb[start: start + n_tok].contiguous(), n_tok, D, m,
                      first[s], s * cap, normalize, R, runs, fmt)
    out = torch.full((S * cap * rb,), 0x5a, dtype=torch.uint8, device=DEV)
    csa.csa_select_and_pad(runs, S, cap, rb, dev(np.array(n_valid, np.int64)), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(S * cap, rb)
    assert sum(n_valid) == n_all
    assert np.array_equal(got[:n_all], whole.cpu().numpy().reshape(-1, rb)[:n_all]), "joined run differs"
    assert not got[n_all:].any(), "padding is not zero"
    return got[:n_all], tok, normalize


@pytest.mark.parametrize("L,cuts,m,D,R,fmt", [
    (3001, [517, 1290, 1294, 2200], 4, 512, 64, csa.SPLIT),    # KV entries; odd cuts, a shard of m tokens
    (2999, [4, 1000, 1603], 4, 128, 0, csa.FP8),               # index keys (no norm, no RoPE)
    (20000, [3000, 9100, 14337], 128, 512, 64, csa.SPLIT),     # HCA
    (4096, [1024, 2048, 3072], 4, 512, 64, csa.SPLIT),         # cuts on block boundaries: nothing carried
    (777, [], 4, 512, 64, csa.SPLIT),                          # one shard
])
def test_cp_shards_join_to_the_unsharded_compression(L, cuts, m, D, R, fmt):
    rows, tok, normalize = _cp_case(L, cuts, m, D, R, fmt, 3000 + L + m)
    n = rows.shape[0]
    xs = torch.from_numpy(tok.x[: n * m]).to(torch.bfloat16).float().numpy().astype(np.float64)
    gs = tok.gate[: n * m].astype(np.float64)
    y = OM.compress_entries(xs, gs, m, 0, eps=EPS, R=R, normalize=normalize)
    tol = _compress_error_bound(xs, gs, m, y, R, normalize)
    if fmt == csa.SPLIT:
        dec = OF.decode_rows(rows, csa.SPLIT, D, R)
        flips = _quant_ok(dec[:, : D - R], y[:, : D - R], csa.FP8, tol[:, : D - R])
        flips += _quant_ok(dec[:, D - R:], y[:, D - R:], csa.BF16, tol[:, D - R:])
    else:
        flips = _quant_ok(OF.decode_rows(rows, fmt, D), y, fmt, tol)
    assert flips <= max(4, y.size // 20000)


def test_select_and_pad_layouts():
    """Shards with no valid row, n_valid past cap (clamped), one shard, and a
    row size that is not a multiple of 16."""
    rng = np.random.default_rng(5)
    for S, cap, rb, nv in [(4, 7, 576, [0, 7, 3, 9]), (1, 5, 4, [2]), (3, 1, 68, [1, 0, 1]), (256, 2, 128, None)]:
        nv = rng.integers(0, cap + 2, size=S) if nv is None else np.array(nv)
        runs = rng.integers(0, 256, size=(S, cap, rb), dtype=np.uint8)
        out = torch.full((S * cap * rb,), 0x33, dtype=torch.uint8, device=DEV)
        csa.csa_select_and_pad(dev(runs.reshape(-1)), S, cap, rb, dev(nv.astype(np.int64)), out)
        torch.cuda.synchronize()
        want = np.concatenate([runs[s, : min(int(nv[s]), cap)] for s in range(S)] + [np.zeros((0, rb), np.uint8)])
        got = out.cpu().numpy().reshape(S * cap, rb)
        assert np.array_equal(got[: len(want)], want)
        assert not got[len(want):].any()

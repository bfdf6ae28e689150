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
    for v in (csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC):
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

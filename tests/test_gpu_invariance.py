"""Batch invariance on the GPU: a token's outputs are bit-identical whatever
it is batched with, wherever it sits in the batch, and whichever attention
variant runs (QbitAI piece on batch invariance: the same token must give the
same bits in any batch; no split-KV, a fixed per-token reduction order)."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, dev, gpu_bytes, upload_decode

pytestmark = pytest.mark.gpu


def _case(cfg, lengths, seed, csa_mode):
    c = synth.WORKLOADS[cfg]
    return synth.decode_inputs(seed, lengths, m=c["m"], H=c["H"], D=c["D"], R=c["R"],
                               n_win=c["n_win"], kv_fmt=c["kv_fmt"], q_fmt=c["q_fmt"],
                               win_fmt=c["win_fmt"], csa=csa_mode, k=c.get("k", 512),
                               idx_fmt=c.get("idx_fmt", csa.FP8), H_I=c.get("H_I", 64),
                               d_I=c.get("d_I", 128))


def _attn(inp, bufs, sel_t, rows, variant):
    """hybrid_attn_decode over the queries `rows` (in that order) of inp; raw output bytes."""
    r = torch.as_tensor(np.asarray(rows, np.int64), device=DEV)
    H, D = inp.H, inp.D
    out_fmt = csa.F32 if inp.q_fmt == csa.F32 else csa.BF16
    rb = csa.row_bytes(out_fmt, D)
    out = gpu_bytes(len(rows) * H * rb)
    idx = sel_t[r].contiguous() if sel_t is not None else None
    csa.hybrid_attn_decode(bufs["q"][r].contiguous(), inp.q_fmt, len(rows), H, D,
                           bufs["q_pos"][r].contiguous(), None, EPS, inp.R, ROPE_BASE, bufs["kv"],
                           inp.kv_fmt, bufs["kv_off"][r].contiguous(), inp.m, idx,
                           inp.k if idx is not None else 0, bufs["win"][r].contiguous(),
                           inp.win_fmt, inp.n_win, bufs["win_len"][r].contiguous(), bufs["sinks"],
                           inp.scale, out, out_fmt, variant)
    return out.view(len(rows), H * rb).cpu().numpy()


@pytest.mark.parametrize("cfg,lengths,csa_mode", [
    ("csa_decode_b16_ctx65536", [65536, 9000, 2051, 130, 5, 40000], True),
    ("hca_decode_b32_ctx262144", [262144, 40000, 128, 127, 9000], False),
    ("csa_decode_fp32_b1_ctx2048", [2048, 300, 7], True),
])
def test_attention_bits_independent_of_batch_and_variant(cfg, lengths, csa_mode):
    inp = _case(cfg, lengths, 70 + synth.WORKLOADS[cfg]["seed"], csa_mode)
    bufs = upload_decode(inp)
    sel = synth.random_selection(np.random.default_rng(3), inp.n_ent, inp.k) if csa_mode else None
    sel_t = dev(sel) if sel is not None else None
    B = inp.B
    base = _attn(inp, bufs, sel_t, list(range(B)), csa.VARIANT_AUTO)
    variants = [csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS]
    for v in variants:
        got = _attn(inp, bufs, sel_t, list(range(B)), v)
        assert np.array_equal(got, base), f"variant {v} changed the bits"
    rng = np.random.default_rng(11)
    for _ in range(3):
        perm = rng.permutation(B)
        got = _attn(inp, bufs, sel_t, list(perm), csa.VARIANT_AUTO)
        assert np.array_equal(got, base[perm]), "batch permutation changed the bits"
    for b in range(B):
        for v in [csa.VARIANT_AUTO] + variants:
            got = _attn(inp, bufs, sel_t, [b], v)
            assert np.array_equal(got[0], base[b]), f"query {b} alone (variant {v}) changed the bits"
    # the same query repeated fills the batch: every copy gets the same bits
    got = _attn(inp, bufs, sel_t, [0] * 64, csa.VARIANT_AUTO)
    assert all(np.array_equal(got[i], base[0]) for i in range(64))


def test_indexer_and_topk_bits_independent_of_batch():
    inp = _case("csa_decode_b16_ctx65536", [65536, 9000, 2051, 130, 5], 81, True)
    bufs = upload_decode(inp)
    B, ld, k = inp.B, int(inp.n_ent.max()), inp.k

    def run(rows):
        r = torch.as_tensor(np.asarray(rows, np.int64), device=DEV)
        sc = torch.full((len(rows), ld), -3.0, dtype=torch.float32, device=DEV)
        csa.indexer_score(bufs["q_idx"][r].contiguous(), bufs["w"][r].contiguous(), len(rows),
                          inp.H_I, inp.d_I, bufs["keys"], inp.idx_fmt,
                          bufs["kv_off"][r].contiguous(), bufs["q_pos"][r].contiguous(), inp.m,
                          sc, ld)
        nv = torch.as_tensor(inp.n_ent[np.asarray(rows)], device=DEV)
        idx = torch.empty((len(rows), k), dtype=torch.int32, device=DEV)
        csa.topk_select(sc, ld, len(rows), nv, k, idx)
        return sc.cpu().numpy(), idx.cpu().numpy()

    s0, i0 = run(list(range(B)))
    perm = np.random.default_rng(5).permutation(B)
    s1, i1 = run(list(perm))
    assert np.array_equal(s1.view(np.uint32), s0[perm].view(np.uint32))
    assert np.array_equal(i1, i0[perm])
    for b in range(B):
        s2, i2 = run([b])
        assert np.array_equal(s2[0].view(np.uint32), s0[b].view(np.uint32))
        assert np.array_equal(i2[0], i0[b])

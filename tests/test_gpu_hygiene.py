"""Memory hygiene of the kernels (a race, or a read of memory a kernel has
not written, makes results depend on stale bytes; batch invariance, QbitAI
piece, asks for the same bits every time).  Every kernel of the path runs
after the LDS of every CU has been filled with a 32-bit pattern
(csa_debug_poison_lds), and the top-k's caller workspace is filled with byte
patterns before its two-pass rows; every result must carry the bits of the
run after a zero fill.  Also the environment switches: CSA_VARIANT forces a
variant (high, low, full) on calls that pass AUTO (the same bits, by
invariance) and CSA_LOG=1
names each launch's choice on stderr."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, dev, gpu_bytes, upload_decode

import test_gpu_fused as fused
import test_gpu_paged as paged
import test_gpu_prefill as prefill

pytestmark = pytest.mark.gpu

PATTERNS = [0x00000000, 0xFFFFFFFF, 0x7F7F7F7F, 0x7FC00000, 0x3C003C00, 0x12345678]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


def _as_bytes(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x).view(np.uint8)


def _same_under_poison(run, what):
    """run() launches the kernels under test and returns their results."""
    ref = None
    for p in PATTERNS:
        csa.debug_poison_lds(p)
        got = [_as_bytes(t) for t in run()]
        torch.cuda.synchronize()
        if ref is None:
            ref = got
            continue
        for j, (a, b) in enumerate(zip(ref, got)):
            assert np.array_equal(a, b), f"{what}: result {j} differs after an LDS fill of {p:#010x}"


def test_compress_score_step_ignores_stale_lds():
    st = fused._case([65536, 9000, 2052, 132, 8, 40000], [True, False, True, True, True, False], 64, csa.FP8, 901)
    _same_under_poison(lambda: fused._run(st, True), "csa_compress_score")
    st4 = fused._case([4096, 260, 8], [True, True, False], 64, csa.MXFP4, 902)
    _same_under_poison(lambda: fused._run(st4, False), "compress + MXFP4 indexer")


def test_fused_topk_ignores_stale_lds():
    """csa_compress_score_topk after every LDS fill: the same scores and sets
    (its LDS bins are cleared at the start of every workgroup)."""
    import test_gpu_score_topk as stk
    st = fused._case([65536, 9000, 2052, 132, 8, 40000], [True, False, True, True, True, False], 64, csa.FP8, 905)
    ws = stk._workspace(st["B"])

    def run():
        _, _, scores, idx = stk._fused(st, 512, ws)
        assert not torch.any(ws != 0).item()
        return scores, idx
    _same_under_poison(run, "csa_compress_score_topk")


def test_topk_ignores_stale_lds_and_workspace():
    rng = np.random.default_rng(903)
    for nq, ld, k, ties in ((16, 16384, 512, 0), (5, 100000, 1024, 3), (3, 5000, 64, 5)):
        sc = dev(synth.random_scores(904 + ld, nq, ld, tie_levels=ties, rng=rng)[0])
        nv = dev(np.array([ld] + [int(x) for x in rng.integers(0, ld, nq - 1)], np.int64))
        need = csa.topk_workspace_bytes(nq, ld, k)

        def run(fill=0):
            idx = torch.full((nq, k), 7, dtype=torch.int32, device=DEV)
            top = torch.full((nq, k), 7.0, dtype=torch.float32, device=DEV)
            ws = torch.full((max(need, 1),), fill, dtype=torch.uint8, device=DEV) if need else None
            csa.topk_select(sc, ld, nq, nv, k, idx, top, workspace=ws)
            return [idx, top]
        _same_under_poison(run, f"topk_select {nq}x{ld} k={k}")
        if need:
            ref = [_as_bytes(t) for t in run(0)]
            for fill in (0xFF, 0x7F, 0x80, 0x01):
                got = [_as_bytes(t) for t in run(fill)]
                assert all(np.array_equal(a, b) for a, b in zip(ref, got)), f"workspace fill {fill:#x} changed it"


@pytest.mark.parametrize("cfg,lengths,csa_mode", [
    ("csa_decode_b16_ctx65536", [65536, 9000, 2051, 130, 5], True),
    ("hca_decode_b32_ctx262144", [262144, 40000, 128, 127], False),
    ("csa_decode_fp32_b1_ctx2048", [2048, 300, 7], True),
])
def test_decode_attention_ignores_stale_lds(cfg, lengths, csa_mode):
    c = synth.WORKLOADS[cfg]
    inp = synth.decode_inputs(905, lengths, m=c["m"], H=c["H"], D=c["D"], R=c["R"], n_win=c["n_win"],
                              kv_fmt=c["kv_fmt"], q_fmt=c["q_fmt"], win_fmt=c["win_fmt"], csa=csa_mode,
                              k=c.get("k", 512), idx_fmt=c.get("idx_fmt", csa.FP8), H_I=c.get("H_I", 64),
                              d_I=c.get("d_I", 128))
    b = upload_decode(inp)
    sel = dev(synth.random_selection(np.random.default_rng(906), inp.n_ent, inp.k)) if csa_mode else None
    out_fmt = csa.F32 if inp.q_fmt == csa.F32 else csa.BF16
    for v in (csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS):
        def run():
            out = gpu_bytes(inp.B * inp.H * csa.row_bytes(out_fmt, inp.D))
            csa.hybrid_attn_decode(b["q"], inp.q_fmt, inp.B, inp.H, inp.D, b["q_pos"], None, EPS, inp.R,
                                   ROPE_BASE, b["kv"], inp.kv_fmt, b["kv_off"], inp.m, sel,
                                   inp.k if csa_mode else 0, b["win"], inp.win_fmt, inp.n_win, b["win_len"],
                                   b["sinks"], inp.scale, out, out_fmt, v)
            return [out]
        _same_under_poison(run, f"hybrid_attn_decode {cfg} variant {v}")


def test_paged_attention_and_prefill_ignore_stale_lds():
    inp = synth.decode_inputs(907, [65536, 9000, 130, 5], m=4, H=16, D=512, R=64, k=512)
    sel = synth.random_selection(np.random.default_rng(908), inp.n_ent, inp.k)
    _same_under_poison(lambda: paged._attn_pair(inp, sel, 32, 909, csa.VARIANT_AUTO, ring=True),
                       "hybrid_attn_decode(_paged)")
    c = prefill._case(910, 3000, 64, 32, 4, 256)
    bufs = prefill._prefill(c, csa.VARIANT_AUTO)[1]
    _same_under_poison(lambda: [prefill._prefill(c, csa.VARIANT_AUTO, bufs)[0]], "hybrid_attn_prefill")


def test_shared_key_indexer_ignores_stale_lds():
    gen = synth.device_generator(911)
    rng = np.random.default_rng(912)
    m, d_I, H_I = 4, 128, 64
    n_a, n_b = 20000, 3000
    keys = synth.device_rows(gen, n_a + n_b, d_I, csa.FP8)
    nq_a, nq_b = 701, 401
    q_pos = dev(np.concatenate([rng.integers(0, n_a * m, nq_a), rng.integers(0, n_b * m, nq_b)]).astype(np.int64))
    key_off = dev(np.concatenate([np.zeros(nq_a), np.full(nq_b, n_a)]).astype(np.int64))
    nq = nq_a + nq_b
    q_idx = synth.device_rows(gen, nq * H_I, d_I, csa.FP8).reshape(nq, H_I, -1)
    w = torch.rand((nq, H_I), generator=gen, device=DEV, dtype=torch.float32)

    def run():
        sc = torch.full((nq, n_a), -7.0, dtype=torch.float32, device=DEV)
        csa.indexer_score(q_idx, w, nq, H_I, d_I, keys, csa.FP8, key_off, q_pos, m, sc, n_a)
        return [sc]
    _same_under_poison(run, "indexer_score (shared-key kernel)")


_CHILD = r"""
import sys, hashlib, torch
sys.path.insert(0, sys.argv[1])
import numpy as np
import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
inp = synth.decode_inputs(913, [65536, 9000, 130], m=4, H=16, D=512, R=64, k=512)
sel = synth.random_selection(np.random.default_rng(914), inp.n_ent, inp.k)
t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
out = torch.empty(inp.B * inp.H * 1024, dtype=torch.uint8, device="cuda:0")
csa.hybrid_attn_decode(t(inp.q), csa.BF16, inp.B, inp.H, 512, t(inp.q_pos), None, 1e-6, 64, 10000.0, t(inp.kv),
                       csa.SPLIT, t(inp.kv_off), 4, t(sel), 512, t(inp.win), csa.BF16, inp.n_win, t(inp.win_len),
                       t(inp.sinks), inp.scale, out, csa.BF16, int(sys.argv[2]))
torch.cuda.synchronize()
print(hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest())
"""


def _child(env_extra, variant):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, str(variant)], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout.strip().splitlines()[-1], r.stderr


def test_variant_and_log_from_the_environment():
    base, _ = _child({"CSA_LOG": "0"}, csa.VARIANT_HIGH_OCC)
    forced, log = _child({"CSA_LOG": "1", "CSA_VARIANT": "low"}, csa.VARIANT_AUTO)
    assert forced == base, "a forced variant changed the bits"
    assert "variant LOW_OCC (CSA_VARIANT)" in log, log[-2000:]
    full, log3 = _child({"CSA_LOG": "1", "CSA_VARIANT": "full"}, csa.VARIANT_AUTO)
    assert full == base, "the FULL_DIMS variant changed the bits"
    assert "variant FULL_DIMS (CSA_VARIANT)" in log3, log3[-2000:]
    kept, log2 = _child({"CSA_LOG": "1", "CSA_VARIANT": "low"}, csa.VARIANT_HIGH_OCC)
    assert kept == base
    assert "variant HIGH_OCC (requested)" in log2, log2[-2000:]

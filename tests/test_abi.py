"""The C ABI without a GPU: the built library loads, exports every function
include/csa.h declares, and rejects bad arguments on the host before any
device work (no compute call runs here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("__")))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_every_declared_function_is_exported(lib):
    names = _declared()
    assert set(names) == set(binding.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"libcsa.so does not export {n}"


def test_version_status_strings_and_row_bytes(lib):
    assert lib.csa_abi_version() == 4
    lib.csa_status_string.restype = ctypes.c_char_p
    for code, name in ((0, b"CSA_OK"), (1, b"CSA_ERR_INVALID_ARG"), (2, b"CSA_ERR_UNSUPPORTED"),
                       (3, b"CSA_ERR_HIP"), (4, b"CSA_ERR_WORKSPACE")):
        assert lib.csa_status_string(code) == name
    lib.csa_row_bytes.restype = ctypes.c_size_t
    for fmt in (csa.F32, csa.BF16, csa.FP8, csa.MXFP4, csa.SPLIT):
        assert lib.csa_row_bytes(fmt, 512, 64) == synth.row_bytes(fmt, 512, 64)
    assert lib.csa_row_bytes(csa.SPLIT, 512, 64) == 576          # 448 FP8 + 64 BF16 dims
    assert lib.csa_row_bytes(csa.MXFP4, 128, 0) == 68             # 64 code bytes + 4 scales
    assert lib.csa_row_bytes(csa.MXFP4, 100, 0) == 0              # not a multiple of 32
    assert lib.csa_row_bytes(99, 512, 64) == 0


def _last_error(lib):
    lib.csa_last_error.restype = ctypes.c_char_p
    return lib.csa_last_error().decode()


def _fake(n=1):
    """A non-null host address: argument checks run before any pointer is used."""
    return ctypes.c_void_p(0x1000 * n)


def test_topk_argument_errors(lib):
    p = _fake()
    for ld, nq, k, want in ((100, 1, 0, INVALID), (100, 1, 4097, INVALID), (0, 1, 8, INVALID),
                            ((1 << 28) + 1, 1, 8, INVALID), (100, -1, 8, INVALID), (100, (1 << 22) + 1, 8, INVALID)):
        st = lib.topk_select(p, ctypes.c_int64(ld), nq, None, k, p, None, None, 0, None)
        assert st == want, (ld, nq, k, st)
        assert "topk_select" in _last_error(lib)
    assert lib.topk_select(None, ctypes.c_int64(100), 1, None, 8, None, None, None, 0, None) == INVALID
    assert lib.topk_select(None, ctypes.c_int64(100), 0, None, 8, None, None, None, 0, None) == OK
    # rows x slices past 2^22 workgroups: rejected before anything is launched
    assert lib.topk_select(p, ctypes.c_int64(1 << 20), 1 << 20, None, 512, p, None, p, 1 << 62, None) == INVALID


WORKSPACE = 4


def test_topk_workspace_contract(lib):
    """Rows up to 33792 scores need no workspace; longer rows need nq * P * k * 8
    bytes of caller memory (P slices of about 16K scores), and a missing, short
    or misaligned workspace is refused with CSA_ERR_WORKSPACE before any launch."""
    wsb = lib.csa_topk_workspace_bytes
    assert wsb(16, 16384, 512) == 0 and wsb(4, 33792, 1024) == 0
    assert wsb(16, 262144, 512) == 16 * 16 * 512 * 8             # P = 16 slices of 16384
    assert wsb(64, 262144, 1024) == 64 * 16 * 1024 * 8            # P = min(16, 16384 / 1024)
    assert wsb(3, 1048576, 512) == 3 * 32 * 512 * 8               # P = 16384 / 512 = 32
    assert wsb(2, 40000, 4096) == 2 * 3 * 4096 * 8                # P = ceil(40000 / 16384)
    assert wsb(0, 262144, 512) == 0 and wsb(4, 262144, 0) == 0    # rejected sizes
    assert csa.topk_workspace_bytes(16, 262144, 512) == wsb(16, 262144, 512)
    p = _fake()
    need = wsb(16, 262144, 512)
    assert lib.topk_select(p, ctypes.c_int64(262144), 16, None, 512, p, None, None, need, None) == WORKSPACE
    assert "workspace" in _last_error(lib)
    assert lib.topk_select(p, ctypes.c_int64(262144), 16, None, 512, p, None, p, need - 1, None) == WORKSPACE
    assert lib.topk_select(p, ctypes.c_int64(262144), 16, None, 512, p, None, ctypes.c_void_p(0x1004), need,
                           None) == WORKSPACE
    lib.csa_status_string.restype = ctypes.c_char_p
    assert lib.csa_status_string(WORKSPACE) == b"CSA_ERR_WORKSPACE"


def test_topk_noalloc_limits(lib):
    """The no-allocation top-k holds 16 MiB of candidates per GPU; larger
    selections and bad arguments are refused on the host, before any device
    call."""
    assert lib.csa_topk_noalloc_max_bytes() == 16 << 20
    p = _fake()
    nq, ld, k = 256, 1 << 20, 4096
    assert lib.csa_topk_workspace_bytes(nq, ld, k) == nq * 4 * k * 8 > 16 << 20
    assert lib.topk_select_noalloc(p, ctypes.c_int64(ld), nq, None, k, p, None, None) == WORKSPACE
    assert "static scratch" in _last_error(lib)
    assert lib.topk_select_noalloc(p, ctypes.c_int64(ld), 4, None, 0, p, None, None) == INVALID
    assert lib.topk_select_noalloc(None, ctypes.c_int64(ld), 4, None, 512, p, None, None) == INVALID
    assert lib.topk_select_noalloc(p, ctypes.c_int64(ld), -1, None, 512, p, None, None) == INVALID
    assert lib.topk_select_noalloc(p, ctypes.c_int64(ld), 0, None, 512, p, None, None) == 0


def test_compress_argument_errors(lib):
    p = _fake()
    base = dict(x=p, x_fmt=csa.F32, gate=p, gate_cols=1, n_tok=8, D=512, m=4, nseg=1, off=p, pos0=p,
                row=p, normalize=1, norm_w=None, eps=1e-6, R=64, base=1e4, out=p, out_fmt=csa.SPLIT)

    def call(**kw):
        a = dict(base, **kw)
        return lib.csa_compress(a["x"], a["x_fmt"], a["gate"], a["gate_cols"], ctypes.c_int64(a["n_tok"]),
                                a["D"], a["m"], a["nseg"], a["off"], a["pos0"], a["row"], a["normalize"],
                                a["norm_w"], ctypes.c_float(a["eps"]), a["R"], ctypes.c_float(a["base"]),
                                a["out"], a["out_fmt"], None)
    assert call(n_tok=7) == INVALID                 # n_tok % m != 0
    assert call(m=0) == INVALID
    assert call(gate_cols=3) == INVALID             # neither 1 nor D
    assert call(R=63) == INVALID                    # odd RoPE dims
    assert call(out_fmt=csa.MXFP4, D=100, R=0) == INVALID
    assert call(R=0) == INVALID                     # SPLIT needs RoPE dims
    assert call(x_fmt=csa.FP8) == INVALID
    assert call(D=8192) == UNSUPPORTED
    assert call(x=None) == INVALID
    assert call(eps=-1.0) == INVALID


def test_compress_batch_argument_errors(lib):
    p = _fake()
    job = binding.CompressJob(x=p.value, x_fmt=csa.F32, gate=p.value, gate_cols=1, n_tok=8, D=512,
                              m=4, nseg=1, seg_tok_off=p.value, seg_pos0=p.value, seg_out_row=p.value,
                              normalize=1, norm_w=None, eps=1e-6, rope_dim=64, rope_base=1e4,
                              out=p.value, out_fmt=csa.SPLIT)
    bad = binding.CompressJob.from_buffer_copy(job)
    bad.m = 0
    arr = (binding.CompressJob * 5)(job, bad, job, job, job)
    for n in (-1, 5):
        assert lib.csa_compress_batch(arr, n, None) == INVALID
        assert "n_jobs" in _last_error(lib)
    assert lib.csa_compress_batch(None, 2, None) == INVALID
    # a failing job stops the call before any launch and is named
    assert lib.csa_compress_batch(arr, 2, None) == INVALID
    assert "job 1" in _last_error(lib)
    assert lib.csa_compress_batch(arr, 0, None) == OK
    empty = binding.CompressJob.from_buffer_copy(job)
    empty.n_tok = 0
    assert lib.csa_compress_batch((binding.CompressJob * 1)(empty), 1, None) == OK


def test_attention_argument_errors(lib):
    p = _fake()

    def call(q_fmt=csa.BF16, kv_fmt=csa.SPLIT, win_fmt=csa.BF16, out_fmt=csa.BF16, D=512, R=64, H=64,
             variant=0, q=p):
        return lib.hybrid_attn_decode(q, q_fmt, 2, H, D, p, None, ctypes.c_float(1e-6), R,
                                      ctypes.c_float(1e4), p, kv_fmt, p, 4, p, 512, p, win_fmt, 128,
                                      p, p, ctypes.c_float(0.04), p, out_fmt, variant, None)
    assert call(kv_fmt=csa.FP8) == UNSUPPORTED       # neither the all-F32 nor the MFMA path
    assert call(D=256) == UNSUPPORTED                # the MFMA path is D = 512, 64 RoPE dims
    assert call(H=40) == UNSUPPORTED                 # heads in tiles of 16
    assert call(q_fmt=csa.F32, kv_fmt=csa.F32, win_fmt=csa.F32, out_fmt=csa.F32, D=640) == UNSUPPORTED
    assert call(variant=7) == INVALID
    assert call(variant=4) == INVALID                # AUTO, HIGH_OCC, LOW_OCC, FULL_DIMS are 0..3
    assert call(q=None) == INVALID
    assert "hybrid_attn_decode" in _last_error(lib)


def test_indexer_argument_errors(lib):
    p = _fake()

    def call(fmt=csa.FP8, H=64, d=128, nq=2, m=4, ld=1024):
        return lib.indexer_score(p, p, nq, H, d, p, fmt, p, p, m, p, ctypes.c_int64(ld), None)
    assert call(fmt=csa.SPLIT) in (INVALID, UNSUPPORTED)
    assert call(d=96) in (INVALID, UNSUPPORTED)      # FP8 / MXFP4 keys are 128-dim
    assert call(H=40) in (INVALID, UNSUPPORTED)
    assert call(m=0) == INVALID
    assert call(ld=0) == INVALID
    assert call(ld=(1 << 24) + 1) == INVALID          # key rows must stay under 2^31 bytes
    assert call(nq=0) == OK


def test_compress_score_argument_errors(lib):
    """csa_compress_score's host checks: those of both calls it stands for,
    plus the shape of the job that writes the indexer keys."""
    p, keys = _fake(), _fake(2)

    def key_job(**kw):
        j = binding.CompressJob(x=p.value, x_fmt=csa.BF16, gate=p.value, gate_cols=1, n_tok=8, D=128,
                                m=4, nseg=2, seg_tok_off=p.value, seg_pos0=p.value, seg_out_row=p.value,
                                normalize=0, norm_w=None, eps=1e-6, rope_dim=0, rope_base=1e4,
                                out=keys.value, out_fmt=csa.FP8)
        for k, v in kw.items():
            setattr(j, k, v)
        return j

    def call(jobs, nq=2, fmt=csa.FP8, H=64, d=128, ld=1024):
        arr = (binding.CompressJob * max(1, len(jobs)))(*jobs)
        return lib.csa_compress_score(arr, len(jobs), p, p, nq, H, d, keys, fmt, p, p, 4, p,
                                      ctypes.c_int64(ld), None)
    for bad in (dict(nseg=1), dict(D=64), dict(out_fmt=csa.MXFP4), dict(rope_dim=2)):
        assert call([key_job(**bad)]) == INVALID, bad
        assert "csa_compress_score" in _last_error(lib)
    assert call([key_job(), key_job()]) == INVALID               # two jobs write `keys`
    assert "both write" in _last_error(lib)
    assert call([key_job(m=0)]) == INVALID                       # the job's own checks
    assert "job 0" in _last_error(lib)
    assert call([key_job()], d=96) == UNSUPPORTED                # the indexer's own checks
    assert call([key_job()], ld=0) == INVALID
    assert lib.csa_compress_score(None, 0, p, p, 0, 64, 128, keys, csa.FP8, p, p, 4, p,
                                  ctypes.c_int64(1024), None) == OK   # nothing to do


def test_compress_score_topk_argument_errors(lib):
    """csa_compress_score_topk's host checks: k, idx, the key format and batch
    size of the one-launch selection, and the zeroed workspace it needs
    (CSA_ERR_WORKSPACE when missing, short or misaligned); nothing is
    launched when a check fails."""
    p = _fake()
    need = lib.csa_score_topk_workspace_bytes(16)
    assert need == 16 * 16640
    assert lib.csa_score_topk_workspace_bytes(0) == 0 and lib.csa_score_topk_workspace_bytes(1024) == 0
    ws = ctypes.c_void_p(1 << 40)                              # 256-byte aligned (never touched)

    def call(nq=16, fmt=csa.FP8, k=512, idx=p, w=ws, nb=need, ld=16384):
        return lib.csa_compress_score_topk(None, 0, p, p, nq, 64, 128, p, fmt, p, p, 4, p, ctypes.c_int64(ld), k,
                                           idx, w, nb, None)
    for k in (0, 4097, -1):
        assert call(k=k) == INVALID, k
        assert "csa_compress_score_topk" in _last_error(lib)
    assert call(idx=None) == INVALID
    assert call(fmt=csa.MXFP4) == UNSUPPORTED
    assert call(nq=1024) == UNSUPPORTED
    assert call(w=None) == WORKSPACE
    assert call(nb=need - 1) == WORKSPACE
    assert call(w=ctypes.c_void_p((1 << 40) + 16)) == WORKSPACE
    assert "aligned" in _last_error(lib)
    assert call(ld=0) == INVALID                               # the indexer's own checks
    assert call(nq=0, w=None, nb=0) == OK                      # nothing to do
    tbl = _fake(3)
    assert lib.csa_compress_score_topk_paged(None, 0, p, p, 2, 64, 128, p, csa.FP8, ctypes.c_int64(1000), tbl,
                                             ctypes.c_int64(2), ctypes.c_int64(4), 32, None, p, 4, p,
                                             ctypes.c_int64(128), 512, p, None, 0, None) == WORKSPACE
    assert "csa_compress_score_topk_paged" in _last_error(lib)


def test_select_and_pad_argument_errors(lib):
    """csa_select_and_pad's host checks (nothing is launched when one fails)."""
    a, b, nv = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 41), _fake()

    def call(S=4, cap=8, rb=576, i=a, o=b, n=nv):
        return lib.csa_select_and_pad(i, S, ctypes.c_int64(cap), ctypes.c_int64(rb), n, o, None)
    for bad in (dict(S=0), dict(S=257), dict(cap=-1), dict(rb=6), dict(rb=0), dict(i=None), dict(n=None),
                dict(o=ctypes.c_void_p((1 << 40) + 1000)), dict(o=ctypes.c_void_p((1 << 41) + 2))):
        assert call(**bad) == INVALID, bad
        assert "csa_select_and_pad" in _last_error(lib)
    assert call(cap=0, i=None, o=None, n=None) == OK             # nothing to do


def test_paged_entry_points_argument_errors(lib):
    """indexer_score_paged / hybrid_attn_{decode,prefill}_paged: block geometry, pool
    size and format checks run on the host before any launch."""
    p, tbl = _fake(), _fake(3)

    def idx(fmt=csa.FP8, pool_rows=1000, bps=10, br=32, d=128):
        return lib.indexer_score_paged(p, p, 2, 64, d, p, fmt, ctypes.c_int64(pool_rows), tbl,
                                       ctypes.c_int64(bps), br, p, 4, p, ctypes.c_int64(1024), None)
    assert idx(br=24) == INVALID                   # not a power of two
    assert idx(br=8) == INVALID                    # below one 16-key MFMA block
    assert idx(bps=0) == INVALID
    assert idx(pool_rows=0) == INVALID
    assert idx(pool_rows=1 << 26) == UNSUPPORTED   # 8 GiB of 128-byte keys: past 32-bit offsets
    assert idx(fmt=csa.F32) == UNSUPPORTED
    assert idx(d=96) == UNSUPPORTED
    assert "indexer_score_paged" in _last_error(lib)

    def idr(nq=2, table_rows=4, qrow=p, br=32):
        return lib.indexer_score_paged_rows(p, p, nq, 64, 128, p, csa.FP8, ctypes.c_int64(1000), tbl,
                                            ctypes.c_int64(table_rows), ctypes.c_int64(10), br, qrow, p, 4, p,
                                            ctypes.c_int64(1024), None)
    assert idr(table_rows=0) == INVALID
    assert idr(table_rows=1 << 32) == INVALID
    assert idr(br=24) == INVALID
    assert idr(nq=5, table_rows=4, qrow=None) == INVALID   # query 4 would read table row 4
    assert "indexer_score_paged_rows" in _last_error(lib)
    assert idr(nq=0) == OK

    def cs(fmt=csa.FP8, table_rows=4, br=32):
        return lib.csa_compress_score_paged(None, 0, p, p, 2, 64, 128, p, fmt, ctypes.c_int64(1000), tbl,
                                            ctypes.c_int64(table_rows), ctypes.c_int64(10), br, p, p, 4, p,
                                            ctypes.c_int64(1024), None)
    assert cs(fmt=csa.F32) == UNSUPPORTED
    assert cs(table_rows=0) == INVALID
    assert cs(br=8) == INVALID
    assert "csa_compress_score_paged" in _last_error(lib)

    def att(q_fmt=csa.BF16, kv_fmt=csa.SPLIT, br=32, bps=10, pool_rows=1000, table=tbl):
        return lib.hybrid_attn_decode_paged(p, q_fmt, 2, 64, 512, p, None, ctypes.c_float(1e-6), 64,
                                            ctypes.c_float(1e4), p, kv_fmt, ctypes.c_int64(pool_rows), table,
                                            ctypes.c_int64(bps), br, 4, p, 512, p, csa.BF16, 128, None, p, p,
                                            ctypes.c_float(0.04), p, csa.BF16, 0, None)
    assert att(br=3) == INVALID
    assert att(bps=0) == INVALID
    assert att(pool_rows=1 << 23) == UNSUPPORTED   # 4.8 GB of 576-byte entries
    assert att(q_fmt=csa.F32, kv_fmt=csa.F32) == UNSUPPORTED
    assert att(table=None) == INVALID
    assert "hybrid_attn_decode_paged" in _last_error(lib)

    def pre(nq=2, q_fmt=csa.BF16, br=32, bps=10, pool_rows=1000, table=tbl, table_rows=4, qrow=p):
        return lib.hybrid_attn_prefill_paged(p, q_fmt, nq, 64, 512, p, None, ctypes.c_float(1e-6), 64,
                                             ctypes.c_float(1e4), p, csa.SPLIT, ctypes.c_int64(pool_rows), table,
                                             ctypes.c_int64(table_rows), ctypes.c_int64(bps), br, qrow, 4, p, 512,
                                             p, csa.BF16, p, p, 128, p, ctypes.c_float(0.04), p, csa.BF16, 0, None)
    assert pre(br=48) == INVALID
    assert pre(bps=0) == INVALID
    assert pre(table_rows=0) == INVALID
    assert pre(table_rows=1 << 32) == INVALID
    assert pre(pool_rows=0) == INVALID
    assert pre(pool_rows=1 << 23) == UNSUPPORTED
    assert pre(q_fmt=csa.F32) == UNSUPPORTED
    assert pre(table=None) == INVALID
    assert pre(nq=5, table_rows=4, qrow=None) == INVALID   # query 4 would read table row 4
    assert "hybrid_attn_prefill_paged" in _last_error(lib)
    assert pre(nq=0) == OK


def test_log_names_errors_on_stderr():
    """CSA_LOG=1 copies every error message to stderr (read once per process)."""
    code = ("import sys, ctypes; sys.path.insert(0, sys.argv[1]); import compressed_sparse_long_csa_amd as c; "
            "lib = c.load_library(); "
            "print(lib.topk_select(None, ctypes.c_int64(100), 1, None, 8, None, None, None, 0, None))")
    for level, shown in (("1", True), ("0", False)):
        r = subprocess.run([sys.executable, "-c", code, ROOT], env=dict(os.environ, CSA_LOG=level),
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        assert r.stdout.strip().splitlines()[-1] == str(INVALID)
        assert ("[csa] error 1: topk_select" in r.stderr) == shown, r.stderr[-2000:]

"""ctypes binding of libcsa (include/csa.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libcsa.so.  torch tensors supply device memory and the current stream.  Each
wrapper checks dtypes, devices and buffer sizes on the host before calling
the C entry point; with check=True it also copies the small index arrays to
the host and verifies that every row the kernels will touch lies inside its
buffer.  The library must be built (python -m compressed_sparse_long_csa_amd.build);
there is no fallback.
"""
import ctypes
import os

import torch

F32, BF16, FP8, MXFP4, SPLIT = 0, 1, 2, 3, 4
VARIANT_AUTO, VARIANT_HIGH_OCC, VARIANT_LOW_OCC, VARIANT_FULL_DIMS = 0, 1, 2, 3
_STATUS = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_UNSUPPORTED", 3: "CSA_ERR_HIP",
           4: "CSA_ERR_WORKSPACE"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libcsa.so")

# exported symbols declared in include/csa.h
EXPORTS = ("csa_abi_version", "csa_status_string", "csa_last_error", "csa_row_bytes",
           "csa_compress", "csa_compress_batch", "csa_compress_score", "csa_compress_score_paged",
           "csa_compress_score_topk", "csa_compress_score_topk_paged", "csa_score_topk_workspace_bytes", "csa_select_and_pad",
           "indexer_score",
           "indexer_score_paged", "indexer_score_paged_rows", "topk_select", "csa_topk_workspace_bytes", "topk_select_noalloc",
           "csa_topk_noalloc_max_bytes", "hybrid_attn_decode",
           "hybrid_attn_decode_paged", "hybrid_attn_prefill", "hybrid_attn_prefill_paged",
           "csa_debug_poison_lds")

_lib = None


class CsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library():
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m compressed_sparse_long_csa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.csa_abi_version.restype = I
    lib.csa_status_string.restype = ctypes.c_char_p
    lib.csa_status_string.argtypes = [I]
    lib.csa_last_error.restype = ctypes.c_char_p
    lib.csa_row_bytes.restype = U
    lib.csa_row_bytes.argtypes = [I, I, I]
    lib.csa_compress.restype = I
    lib.csa_compress.argtypes = [P, I, P, I, I64, I, I, I, P, P, P, I, P, F, I, F, P, I, P]
    lib.csa_compress_batch.restype = I
    lib.csa_compress_batch.argtypes = [ctypes.POINTER(CompressJob), I, P]
    lib.csa_compress_score.restype = I
    lib.csa_compress_score.argtypes = [ctypes.POINTER(CompressJob), I, P, P, I, I, I, P, I, P, P, I, P,
                                       I64, P]
    lib.csa_compress_score_paged.restype = I
    lib.csa_compress_score_paged.argtypes = [ctypes.POINTER(CompressJob), I, P, P, I, I, I, P, I, I64, P, I64, I64, I,
                                             P, P, I, P, I64, P]
    lib.csa_compress_score_topk.restype = I
    lib.csa_compress_score_topk.argtypes = [ctypes.POINTER(CompressJob), I, P, P, I, I, I, P, I, P, P, I, P,
                                            I64, I, P, P, U, P]
    lib.csa_compress_score_topk_paged.restype = I
    lib.csa_compress_score_topk_paged.argtypes = [ctypes.POINTER(CompressJob), I, P, P, I, I, I, P, I, I64, P, I64,
                                                  I64, I, P, P, I, P, I64, I, P, P, U, P]
    lib.csa_select_and_pad.restype = I
    lib.csa_select_and_pad.argtypes = [P, I, I64, I64, P, P, P]
    lib.csa_score_topk_workspace_bytes.restype = U
    lib.csa_score_topk_workspace_bytes.argtypes = [I]
    lib.indexer_score_paged.restype = I
    lib.indexer_score_paged.argtypes = [P, P, I, I, I, P, I, I64, P, I64, I, P, I, P, I64, P]
    lib.indexer_score_paged_rows.restype = I
    lib.indexer_score_paged_rows.argtypes = [P, P, I, I, I, P, I, I64, P, I64, I64, I, P, P, I, P, I64, P]
    lib.hybrid_attn_decode_paged.restype = I
    lib.hybrid_attn_decode_paged.argtypes = [P, I, I, I, I, P, P, F, I, F, P, I, I64, P, I64, I, I, P, I, P, I, I,
                                             P, P, P, F, P, I, I, P]
    lib.indexer_score.restype = I
    lib.indexer_score.argtypes = [P, P, I, I, I, P, I, P, P, I, P, I64, P]
    lib.topk_select.restype = I
    lib.topk_select.argtypes = [P, I64, I, P, I, P, P, P, U, P]
    lib.csa_topk_workspace_bytes.restype = U
    lib.csa_topk_workspace_bytes.argtypes = [I, I64, I]
    lib.topk_select_noalloc.restype = I
    lib.topk_select_noalloc.argtypes = [P, I64, I, P, I, P, P, P]
    lib.csa_topk_noalloc_max_bytes.restype = U
    lib.csa_topk_noalloc_max_bytes.argtypes = []
    lib.hybrid_attn_decode.restype = I
    lib.hybrid_attn_decode.argtypes = [P, I, I, I, I, P, P, F, I, F, P, I, P, I, P, I, P, I, I, P,
                                       P, F, P, I, I, P]
    lib.hybrid_attn_prefill.restype = I
    lib.hybrid_attn_prefill.argtypes = [P, I, I, I, I, P, P, F, I, F, P, I, P, I, P, I, P, I, P,
                                        P, I, P, F, P, I, I, P]
    lib.hybrid_attn_prefill_paged.restype = I
    lib.hybrid_attn_prefill_paged.argtypes = [P, I, I, I, I, P, P, F, I, F, P, I, I64, P, I64, I64, I, P, I, P, I,
                                              P, I, P, P, I, P, F, P, I, I, P]
    lib.csa_debug_poison_lds.restype = I
    lib.csa_debug_poison_lds.argtypes = [ctypes.c_uint32, P]
    _lib = lib
    return lib


def row_bytes(fmt, D, R=0):
    return {F32: 4 * D, BF16: 2 * D, FP8: D, MXFP4: D // 2 + D // 32, SPLIT: (D - R) + 2 * R}[fmt]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, min_bytes=None, min_numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {min_bytes}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {min_numel}")


def _check(status):
    if status != 0:
        raise CsaError(status, load_library().csa_last_error().decode())


def _host(t):
    return t.detach().to("cpu")


# ------------------------------------------------------------------ entry points
def _compress_checks(x, x_fmt, gate, gate_cols, n_tok, D, m, nseg, seg_tok_off, seg_pos0,
                     seg_out_row, norm_w, rope_dim, out, out_fmt, check):
    _need(x, "x", min_bytes=n_tok * row_bytes(x_fmt, D))
    _need(gate, "gate", torch.float32, min_numel=n_tok * gate_cols)
    for t, nm, n in ((seg_tok_off, "seg_tok_off", nseg + 1), (seg_pos0, "seg_pos0", nseg),
                     (seg_out_row, "seg_out_row", nseg)):
        _need(t, nm, torch.int64, min_numel=n)
    _need(norm_w, "norm_w", torch.float32, min_numel=D, allow_none=True)
    _need(out, "out")
    if check and n_tok > 0:
        off = _host(seg_tok_off)[: nseg + 1]
        rows = _host(seg_out_row)[:nseg]
        nent = (off[1:] - off[:-1]) // m
        if off[0] != 0 or off[-1] != n_tok or bool((off[1:] < off[:-1]).any()):
            raise ValueError("seg_tok_off must start at 0, end at n_tok and not decrease")
        need_rows = int((rows + nent).max()) if nseg else 0
        if int(rows.min()) < 0 or out.numel() * out.element_size() < need_rows * row_bytes(out_fmt, D, rope_dim):
            raise ValueError("out is too small for the rows the segments write")


def csa_compress(x, x_fmt, gate, gate_cols, n_tok, D, m, nseg, seg_tok_off, seg_pos0,
                 seg_out_row, normalize, norm_w, eps, rope_dim, rope_base, out, out_fmt,
                 stream=None, check=True):
    lib = load_library()
    _compress_checks(x, x_fmt, gate, gate_cols, n_tok, D, m, nseg, seg_tok_off, seg_pos0,
                     seg_out_row, norm_w, rope_dim, out, out_fmt, check)
    _check(lib.csa_compress(_ptr(x), x_fmt, _ptr(gate), gate_cols, n_tok, D, m, nseg,
                            _ptr(seg_tok_off), _ptr(seg_pos0), _ptr(seg_out_row), int(normalize),
                            _ptr(norm_w), eps, rope_dim, rope_base, _ptr(out), out_fmt,
                            _stream(stream)))


class CompressJob(ctypes.Structure):
    """struct csa_compress_job (include/csa.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("x_fmt", ctypes.c_int), ("gate", ctypes.c_void_p),
                ("gate_cols", ctypes.c_int), ("n_tok", ctypes.c_int64), ("D", ctypes.c_int),
                ("m", ctypes.c_int), ("nseg", ctypes.c_int), ("seg_tok_off", ctypes.c_void_p),
                ("seg_pos0", ctypes.c_void_p), ("seg_out_row", ctypes.c_void_p),
                ("normalize", ctypes.c_int), ("norm_w", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("rope_dim", ctypes.c_int), ("rope_base", ctypes.c_float), ("out", ctypes.c_void_p),
                ("out_fmt", ctypes.c_int)]


COMPRESS_JOB_FIELDS = ("x", "x_fmt", "gate", "gate_cols", "n_tok", "D", "m", "nseg", "seg_tok_off",
                       "seg_pos0", "seg_out_row", "normalize", "norm_w", "eps", "rope_dim",
                       "rope_base", "out", "out_fmt")
MAX_COMPRESS_JOBS = 4


def _job_array(jobs, check):
    arr = (CompressJob * max(1, len(jobs)))()
    for i, j in enumerate(jobs):
        _compress_checks(j["x"], j["x_fmt"], j["gate"], j["gate_cols"], j["n_tok"], j["D"], j["m"],
                         j["nseg"], j["seg_tok_off"], j["seg_pos0"], j["seg_out_row"], j["norm_w"],
                         j["rope_dim"], j["out"], j["out_fmt"], check)
        c = arr[i]
        for f in COMPRESS_JOB_FIELDS:
            v = j[f]
            if isinstance(v, torch.Tensor):
                v = v.data_ptr()
            elif v is None:
                v = None
            setattr(c, f, int(v) if f == "normalize" else v)
    return arr


def csa_compress_batch(jobs, stream=None, check=True):
    """jobs: sequence of dicts with csa_compress's arguments (COMPRESS_JOB_FIELDS)."""
    lib = load_library()
    _check(lib.csa_compress_batch(_job_array(jobs, check), len(jobs), _stream(stream)))


def csa_compress_score(jobs, q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld,
                       stream=None, check=True):
    """csa_compress_batch(jobs) then indexer_score(...), in one launch where it can."""
    lib = load_library()
    arr = _job_array(jobs, check)
    _indexer_checks(q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld, check)
    _check(lib.csa_compress_score(arr, len(jobs), _ptr(q_idx), _ptr(w), nq, n_heads, d_idx, _ptr(keys), fmt,
                                  _ptr(key_off), _ptr(q_pos), m, _ptr(scores), ld, _stream(stream)))


def csa_compress_score_paged(jobs, q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table, table_rows,
                             blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld, stream=None, check=True):
    """csa_compress_batch(jobs) then indexer_score_paged_rows(...), in one launch where it can."""
    lib = load_library()
    arr = _job_array(jobs, check)
    rb = row_bytes(fmt, d_idx)
    _need(q_idx, "q_idx", min_bytes=nq * n_heads * rb)
    _need(w, "w", torch.float32, min_numel=nq * n_heads)
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    _paged_checks(block_table, nq, blocks_per_seq, block_rows, key_pool, pool_rows, rb, q_pos, m, ld, check,
                  table_rows=table_rows, q_block_row=q_block_row)
    _check(lib.csa_compress_score_paged(arr, len(jobs), _ptr(q_idx), _ptr(w), nq, n_heads, d_idx, _ptr(key_pool),
                                        fmt, pool_rows, _ptr(block_table), table_rows, blocks_per_seq, block_rows,
                                        _ptr(q_block_row), _ptr(q_pos), m, _ptr(scores), ld, _stream(stream)))


def csa_select_and_pad(runs, n_shards, cap, row_bytes, n_valid, out, stream=None, check=True):
    """runs: device buffer of n_shards * cap rows of row_bytes; n_valid: int64 [n_shards]
    (device); out: n_shards * cap rows -- the valid rows in shard order, then zeros."""
    lib = load_library()
    if check:
        _need(runs, "runs", min_bytes=n_shards * cap * row_bytes)
        _need(out, "out", min_bytes=n_shards * cap * row_bytes)
        _need(n_valid, "n_valid", torch.int64, min_numel=n_shards)
    _check(lib.csa_select_and_pad(_ptr(runs), n_shards, cap, row_bytes, _ptr(n_valid), _ptr(out), _stream(stream)))


def score_topk_workspace_bytes(nq):
    """Device bytes of zeroed workspace csa_compress_score_topk needs for nq queries."""
    return int(load_library().csa_score_topk_workspace_bytes(nq))


def _score_topk_ws(workspace, nq, k, idx, device):
    _need(idx, "idx", torch.int32, min_numel=nq * k)
    if workspace is None:                  # a fresh zeroed workspace for this call
        workspace = torch.zeros(max(1, score_topk_workspace_bytes(nq)), dtype=torch.uint8, device=device)
    _need(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def csa_compress_score_topk(jobs, q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld, k, idx,
                            workspace=None, stream=None, check=True):
    """csa_compress_score(...) then topk_select(scores, ...) in one launch.  workspace:
    a uint8 device tensor of score_topk_workspace_bytes(nq) bytes, zero before its first
    use (the call leaves it zero); None takes a fresh zeroed one for this call."""
    lib = load_library()
    arr = _job_array(jobs, check)
    _indexer_checks(q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld, check)
    workspace, ws_bytes = _score_topk_ws(workspace, nq, k, idx, scores.device)
    _check(lib.csa_compress_score_topk(arr, len(jobs), _ptr(q_idx), _ptr(w), nq, n_heads, d_idx, _ptr(keys), fmt,
                                       _ptr(key_off), _ptr(q_pos), m, _ptr(scores), ld, k, _ptr(idx),
                                       _ptr(workspace), ws_bytes, _stream(stream)))


def csa_compress_score_topk_paged(jobs, q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table,
                                  table_rows, blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld, k, idx,
                                  workspace=None, stream=None, check=True):
    """csa_compress_score_paged(...) then topk_select(scores, ...) in one launch."""
    lib = load_library()
    arr = _job_array(jobs, check)
    rb = row_bytes(fmt, d_idx)
    _need(q_idx, "q_idx", min_bytes=nq * n_heads * rb)
    _need(w, "w", torch.float32, min_numel=nq * n_heads)
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    _paged_checks(block_table, nq, blocks_per_seq, block_rows, key_pool, pool_rows, rb, q_pos, m, ld, check,
                  table_rows=table_rows, q_block_row=q_block_row)
    workspace, ws_bytes = _score_topk_ws(workspace, nq, k, idx, scores.device)
    _check(lib.csa_compress_score_topk_paged(arr, len(jobs), _ptr(q_idx), _ptr(w), nq, n_heads, d_idx,
                                             _ptr(key_pool), fmt, pool_rows, _ptr(block_table), table_rows,
                                             blocks_per_seq, block_rows, _ptr(q_block_row), _ptr(q_pos), m,
                                             _ptr(scores), ld, k, _ptr(idx), _ptr(workspace), ws_bytes,
                                             _stream(stream)))


def indexer_score(q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld,
                  stream=None, check=True):
    lib = load_library()
    _indexer_checks(q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld, check)
    _check(lib.indexer_score(_ptr(q_idx), _ptr(w), nq, n_heads, d_idx, _ptr(keys), fmt,
                             _ptr(key_off), _ptr(q_pos), m, _ptr(scores), ld, _stream(stream)))


def _paged_checks(table, nq, blocks_per_seq, block_rows, pool, pool_rows, rb, q_pos, m, ld, check,
                  table_rows=None, q_block_row=None):
    """Host-side checks of a block table: its shape, and with check=True that
    every block a query uses is inside the pool.  Query i reads table row
    q_block_row[i] (None: row i) of table_rows rows (None: nq)."""
    table_rows = nq if table_rows is None else table_rows
    _need(table, "block_table", torch.int32, min_numel=table_rows * blocks_per_seq)
    _need(pool, "pool", min_bytes=pool_rows * rb)
    _need(q_block_row, "q_block_row", torch.int32, min_numel=nq, allow_none=True)
    if check and nq > 0:
        N = torch.clamp((_host(q_pos)[:nq] + 1) // m, max=ld)
        if int(N.max()) > blocks_per_seq * block_rows:
            raise ValueError("a query sees more rows than its block-table row holds")
        t = _host(table)[: table_rows * blocks_per_seq].view(table_rows, blocks_per_seq)
        rows = torch.arange(nq) if q_block_row is None else _host(q_block_row)[:nq].long()
        if int(rows.min()) < 0 or int(rows.max()) >= table_rows:
            raise ValueError("a q_block_row entry is outside the block table")
        nb = (N + block_rows - 1) // block_rows
        for i in range(nq):
            used = t[int(rows[i]), : int(nb[i])]
            if used.numel() and (int(used.min()) < 0 or (int(used.max()) + 1) * block_rows > pool_rows):
                raise ValueError(f"query {i} uses a block outside the pool")


def indexer_score_paged(q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table, blocks_per_seq,
                        block_rows, q_pos, m, scores, ld, stream=None, check=True):
    lib = load_library()
    rb = row_bytes(fmt, d_idx)
    _need(q_idx, "q_idx", min_bytes=nq * n_heads * rb)
    _need(w, "w", torch.float32, min_numel=nq * n_heads)
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    _paged_checks(block_table, nq, blocks_per_seq, block_rows, key_pool, pool_rows, rb, q_pos, m, ld, check)
    _check(lib.indexer_score_paged(_ptr(q_idx), _ptr(w), nq, n_heads, d_idx, _ptr(key_pool), fmt, pool_rows,
                                   _ptr(block_table), blocks_per_seq, block_rows, _ptr(q_pos), m, _ptr(scores),
                                   ld, _stream(stream)))


def indexer_score_paged_rows(q_idx, w, nq, n_heads, d_idx, key_pool, fmt, pool_rows, block_table, table_rows,
                             blocks_per_seq, block_rows, q_block_row, q_pos, m, scores, ld, stream=None, check=True):
    lib = load_library()
    rb = row_bytes(fmt, d_idx)
    _need(q_idx, "q_idx", min_bytes=nq * n_heads * rb)
    _need(w, "w", torch.float32, min_numel=nq * n_heads)
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    _paged_checks(block_table, nq, blocks_per_seq, block_rows, key_pool, pool_rows, rb, q_pos, m, ld, check,
                  table_rows=table_rows, q_block_row=q_block_row)
    _check(lib.indexer_score_paged_rows(_ptr(q_idx), _ptr(w), nq, n_heads, d_idx, _ptr(key_pool), fmt, pool_rows,
                                        _ptr(block_table), table_rows, blocks_per_seq, block_rows,
                                        _ptr(q_block_row), _ptr(q_pos), m, _ptr(scores), ld, _stream(stream)))


def _indexer_checks(q_idx, w, nq, n_heads, d_idx, keys, fmt, key_off, q_pos, m, scores, ld, check):
    rb = row_bytes(fmt, d_idx)
    _need(q_idx, "q_idx", min_bytes=nq * n_heads * rb)
    _need(w, "w", torch.float32, min_numel=nq * n_heads)
    _need(keys, "keys")
    _need(key_off, "key_off", torch.int64, min_numel=nq)
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    if check and nq > 0:
        N = (_host(q_pos)[:nq] + 1) // m
        N = torch.clamp(N, max=ld)
        end = _host(key_off)[:nq] + N
        if int(_host(key_off)[:nq].min()) < 0 or int(end.max()) * rb > keys.numel() * keys.element_size():
            raise ValueError("a query's visible keys run past the end of `keys`")


def topk_workspace_bytes(nq, ld, k):
    """Device bytes topk_select needs as workspace for these sizes (0: none)."""
    return int(load_library().csa_topk_workspace_bytes(nq, ld, k))


def topk_select(scores, ld, nq, n_valid, k, idx, top_scores=None, stream=None, check=True, workspace=None):
    """workspace: a uint8 device tensor of at least topk_workspace_bytes(nq, ld, k)
    bytes; when None and one is needed, a fresh one is taken from torch's
    allocator for this call (calls that may overlap must not share one)."""
    lib = load_library()
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    _need(n_valid, "n_valid", torch.int64, min_numel=nq, allow_none=True)
    _need(idx, "idx", torch.int32, min_numel=nq * k)
    _need(top_scores, "top_scores", torch.float32, min_numel=nq * k, allow_none=True)
    ws_need = int(lib.csa_topk_workspace_bytes(nq, ld, k))
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=scores.device)
    _need(workspace, "workspace", allow_none=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.topk_select(_ptr(scores), ld, nq, _ptr(n_valid), k, _ptr(idx), _ptr(top_scores),
                           _ptr(workspace), ws_bytes, _stream(stream)))


def topk_noalloc_max_bytes():
    """Size of topk_select_noalloc's static candidate array (per GPU)."""
    return int(load_library().csa_topk_noalloc_max_bytes())


def topk_select_noalloc(scores, ld, nq, n_valid, k, idx, top_scores=None, stream=None):
    """topk_select without a workspace: the library's static per-GPU array holds
    the candidates, so nothing is allocated.  Calls that may overlap on one GPU
    race on that array."""
    lib = load_library()
    _need(scores, "scores", torch.float32, min_numel=nq * ld)
    _need(n_valid, "n_valid", torch.int64, min_numel=nq, allow_none=True)
    _need(idx, "idx", torch.int32, min_numel=nq * k)
    _need(top_scores, "top_scores", torch.float32, min_numel=nq * k, allow_none=True)
    _check(lib.topk_select_noalloc(_ptr(scores), ld, nq, _ptr(n_valid), k, _ptr(idx), _ptr(top_scores),
                                   _stream(stream)))


def _attn_checks(q, q_fmt, nq, H, D, q_pos, q_norm_w, kv, kv_fmt, kv_off, m, idx, k, sinks, out,
                 out_fmt, rope_dim, check):
    _need(q, "q", min_bytes=nq * H * row_bytes(q_fmt, D, rope_dim))
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(q_norm_w, "q_norm_w", torch.float32, min_numel=D, allow_none=True)
    _need(kv, "kv")
    _need(kv_off, "kv_off", torch.int64, min_numel=nq)
    _need(idx, "idx", torch.int32, min_numel=nq * k, allow_none=True)
    _need(sinks, "sinks", torch.float32, min_numel=H)
    _need(out, "out", min_bytes=nq * H * row_bytes(out_fmt, D, rope_dim))
    if check and nq > 0:
        N = (_host(q_pos)[:nq] + 1) // m
        end = _host(kv_off)[:nq] + N
        if int(_host(kv_off)[:nq].min()) < 0 or \
                int(end.max()) * row_bytes(kv_fmt, D, rope_dim) > kv.numel() * kv.element_size():
            raise ValueError("a query's visible entries run past the end of `kv`")


def hybrid_attn_decode(q, q_fmt, B, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv, kv_fmt,
                       kv_off, m, idx, k, win, win_fmt, n_win, win_len, sinks, scale, out, out_fmt,
                       variant=VARIANT_AUTO, stream=None, check=True):
    lib = load_library()
    _attn_checks(q, q_fmt, B, H, D, q_pos, q_norm_w, kv, kv_fmt, kv_off, m, idx, k, sinks, out,
                 out_fmt, rope_dim, check)
    if n_win > 0:
        _need(win, "win", min_bytes=B * n_win * row_bytes(win_fmt, D, rope_dim))
        _need(win_len, "win_len", torch.int32, min_numel=B)
    _check(lib.hybrid_attn_decode(_ptr(q), q_fmt, B, H, D, _ptr(q_pos), _ptr(q_norm_w), eps,
                                  rope_dim, rope_base, _ptr(kv), kv_fmt, _ptr(kv_off), m, _ptr(idx),
                                  k, _ptr(win), win_fmt, n_win, _ptr(win_len), _ptr(sinks), scale,
                                  _ptr(out), out_fmt, variant, _stream(stream)))


def hybrid_attn_decode_paged(q, q_fmt, B, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv_pool, kv_fmt,
                             pool_rows, block_table, blocks_per_seq, block_rows, m, idx, k, win, win_fmt, n_win,
                             win_len, sinks, scale, out, out_fmt, variant=VARIANT_AUTO, stream=None, check=True,
                             win_start=None):
    lib = load_library()
    rb = row_bytes(kv_fmt, D, rope_dim)
    _need(q, "q", min_bytes=B * H * row_bytes(q_fmt, D, rope_dim))
    _need(q_pos, "q_pos", torch.int64, min_numel=B)
    _need(q_norm_w, "q_norm_w", torch.float32, min_numel=D, allow_none=True)
    _need(idx, "idx", torch.int32, min_numel=B * k, allow_none=True)
    _need(sinks, "sinks", torch.float32, min_numel=H)
    _need(out, "out", min_bytes=B * H * row_bytes(out_fmt, D, rope_dim))
    _paged_checks(block_table, B, blocks_per_seq, block_rows, kv_pool, pool_rows, rb, q_pos, m, 1 << 62, check)
    if n_win > 0:
        _need(win, "win", min_bytes=B * n_win * row_bytes(win_fmt, D, rope_dim))
        _need(win_len, "win_len", torch.int32, min_numel=B)
        _need(win_start, "win_start", torch.int32, min_numel=B, allow_none=True)
    _check(lib.hybrid_attn_decode_paged(_ptr(q), q_fmt, B, H, D, _ptr(q_pos), _ptr(q_norm_w), eps, rope_dim,
                                        rope_base, _ptr(kv_pool), kv_fmt, pool_rows, _ptr(block_table),
                                        blocks_per_seq, block_rows, m, _ptr(idx), k, _ptr(win), win_fmt, n_win,
                                        _ptr(win_start), _ptr(win_len), _ptr(sinks), scale, _ptr(out), out_fmt,
                                        variant, _stream(stream)))


def hybrid_attn_prefill(q, q_fmt, nq, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv, kv_fmt,
                        kv_off, m, idx, k, tok, tok_fmt, tok_off, tok_pos0, n_win, sinks, scale,
                        out, out_fmt, variant=VARIANT_AUTO, stream=None, check=True):
    lib = load_library()
    _attn_checks(q, q_fmt, nq, H, D, q_pos, q_norm_w, kv, kv_fmt, kv_off, m, idx, k, sinks, out,
                 out_fmt, rope_dim, check)
    if n_win > 0:
        _need(tok, "tok")
        _need(tok_off, "tok_off", torch.int64, min_numel=nq)
        _need(tok_pos0, "tok_pos0", torch.int64, min_numel=nq)
        if check and nq > 0:
            p = _host(q_pos)[:nq]
            last = _host(tok_off)[:nq] + (p - _host(tok_pos0)[:nq])
            if int(last.max()) + 1 > (tok.numel() * tok.element_size()) // row_bytes(tok_fmt, D, rope_dim):
                raise ValueError("a query's window runs past the end of `tok`")
    _check(lib.hybrid_attn_prefill(_ptr(q), q_fmt, nq, H, D, _ptr(q_pos), _ptr(q_norm_w), eps,
                                   rope_dim, rope_base, _ptr(kv), kv_fmt, _ptr(kv_off), m,
                                   _ptr(idx), k, _ptr(tok), tok_fmt, _ptr(tok_off), _ptr(tok_pos0),
                                   n_win, _ptr(sinks), scale, _ptr(out), out_fmt, variant,
                                   _stream(stream)))


def hybrid_attn_prefill_paged(q, q_fmt, nq, H, D, q_pos, q_norm_w, eps, rope_dim, rope_base, kv_pool, kv_fmt,
                              pool_rows, block_table, table_rows, blocks_per_seq, block_rows, q_block_row, m, idx,
                              k, tok, tok_fmt, tok_off, tok_pos0, n_win, sinks, scale, out, out_fmt,
                              variant=VARIANT_AUTO, stream=None, check=True):
    lib = load_library()
    rb = row_bytes(kv_fmt, D, rope_dim)
    _need(q, "q", min_bytes=nq * H * row_bytes(q_fmt, D, rope_dim))
    _need(q_pos, "q_pos", torch.int64, min_numel=nq)
    _need(q_norm_w, "q_norm_w", torch.float32, min_numel=D, allow_none=True)
    _need(idx, "idx", torch.int32, min_numel=nq * k, allow_none=True)
    _need(sinks, "sinks", torch.float32, min_numel=H)
    _need(out, "out", min_bytes=nq * H * row_bytes(out_fmt, D, rope_dim))
    _paged_checks(block_table, nq, blocks_per_seq, block_rows, kv_pool, pool_rows, rb, q_pos, m, 1 << 62, check,
                  table_rows=table_rows, q_block_row=q_block_row)
    if n_win > 0:
        _need(tok, "tok")
        _need(tok_off, "tok_off", torch.int64, min_numel=nq)
        _need(tok_pos0, "tok_pos0", torch.int64, min_numel=nq)
        if check and nq > 0:
            p = _host(q_pos)[:nq]
            last = _host(tok_off)[:nq] + (p - _host(tok_pos0)[:nq])
            if int(last.max()) + 1 > (tok.numel() * tok.element_size()) // row_bytes(tok_fmt, D, rope_dim):
                raise ValueError("a query's window runs past the end of `tok`")
    _check(lib.hybrid_attn_prefill_paged(_ptr(q), q_fmt, nq, H, D, _ptr(q_pos), _ptr(q_norm_w), eps, rope_dim,
                                         rope_base, _ptr(kv_pool), kv_fmt, pool_rows, _ptr(block_table),
                                         table_rows, blocks_per_seq, block_rows, _ptr(q_block_row), m, _ptr(idx),
                                         k, _ptr(tok), tok_fmt, _ptr(tok_off), _ptr(tok_pos0), n_win,
                                         _ptr(sinks), scale, _ptr(out), out_fmt, variant, _stream(stream)))


def debug_poison_lds(pattern, stream=None):
    """Fill every CU's LDS with the 32-bit pattern (a test diagnostic)."""
    _check(load_library().csa_debug_poison_lds(pattern & 0xffffffff, _stream(stream)))

"""topk_select_noalloc (the top-k entry point that allocates nothing and keeps
its candidates in the library's static per-GPU array) against topk_select with
a caller workspace: the same bits, on consecutive calls of decreasing size."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from oracle import method as OM

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


def _dev(a):
    return torch.as_tensor(a).to(DEV)


def _pair(seed, nq, ld, lens, k):
    """Both entry points on the same rows; returns (noalloc, with workspace)."""
    s, nv = synth.random_scores(seed, nq, ld, lens, 0)
    S, NV = _dev(s), _dev(nv)
    ref_i = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
    ref_s = torch.full((nq, k), 7.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, csa.topk_workspace_bytes(nq, ld, k)), dtype=torch.uint8, device=DEV)
    csa.topk_select(S, ld, nq, NV, k, ref_i, ref_s, workspace=ws)
    got_i = torch.full((nq, k), -9, dtype=torch.int32, device=DEV)
    got_s = torch.full((nq, k), 9.0, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    csa.topk_select_noalloc(S, ld, nq, NV, k, got_i, got_s)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return s, nv, (got_i, got_s), (ref_i, ref_s)


def test_noalloc_matches_workspace_path_on_two_calls():
    k1, k2 = 1024, 512
    # first call: long ragged rows, two passes through the static array
    # (8 rows x 16 slices x 1024 candidates)
    assert 0 < csa.topk_workspace_bytes(8, 262144, k1) <= csa.topk_noalloc_max_bytes()
    s, nv, got, ref = _pair(91, 8, 262144, [262144] * 5 + [150000, 40000, 900], k1)
    assert torch.equal(got[0], ref[0])
    assert torch.equal(got[1], ref[1])
    for i in (0, 6, 7):
        want = OM.top_k(s[i, : nv[i]].astype(np.float64), k1)
        assert np.array_equal(got[0].cpu().numpy()[i, : len(want)], want)
        assert np.all(got[0].cpu().numpy()[i, len(want):] == -1)
    # second call, smaller: fewer rows, fewer slices, another k; the array
    # still holds the first call's candidates
    assert 0 < csa.topk_workspace_bytes(3, 50000, k2) < csa.topk_workspace_bytes(8, 262144, k1)
    s, nv, got, ref = _pair(92, 3, 50000, [50000, 34000, 20], k2)
    assert torch.equal(got[0], ref[0])
    assert torch.equal(got[1], ref[1])
    for i in range(3):
        want = OM.top_k(s[i, : nv[i]].astype(np.float64), k2)
        assert np.array_equal(got[0].cpu().numpy()[i, : len(want)], want)


def test_noalloc_short_rows_and_limit():
    # one-pass rows need no scratch
    assert csa.topk_workspace_bytes(4, 16384, 512) == 0
    _, _, got, ref = _pair(93, 4, 16384, [16384, 9000, 511, 0], 512)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    # beyond the static array: refused before anything is enqueued
    nq, ld, k = 256, 1 << 20, 4096
    assert csa.topk_workspace_bytes(nq, ld, k) > csa.topk_noalloc_max_bytes()
    scores = torch.zeros(16, dtype=torch.float32, device=DEV)
    out = torch.full((16,), -7, dtype=torch.int32, device=DEV)
    lib = csa.load_library()
    st = lib.topk_select_noalloc(scores.data_ptr(), ld, nq, None, k, out.data_ptr(), None, None)
    assert csa.binding._STATUS.get(st) == "CSA_ERR_WORKSPACE", lib.csa_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == -7)

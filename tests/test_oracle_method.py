"""Pins for the oracle's compressor, RMSNorm, partial RoPE, indexer and top-k."""
import json
import math
import os

import numpy as np

from oracle import method as M

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- compressor
def test_compress_hand_worked_example():
    g = _gold("compress_worked_example.json")
    C = M.compress_blocks(np.array(g["x"]), np.array(g["gate"]), g["m"])
    assert np.allclose(C[0], g["entry"], rtol=0, atol=1e-15)
    y = M.rms_norm(C, eps=0.0)
    assert np.allclose(y[0], np.array(g["entry"]) / math.sqrt(g["rms_sq"]), atol=1e-15)


def test_compress_equal_gates_is_block_mean():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 16))
    for m in (1, 2, 4, 16):
        C = M.compress_blocks(x, np.full((64, 1), 0.7), m)
        assert np.allclose(C, x.reshape(64 // m, m, 16).mean(axis=1), atol=1e-14)


def test_compress_m1_identity_and_constant_input():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((8, 5))
    g = rng.standard_normal((8, 1))
    assert np.array_equal(M.compress_blocks(x, g, 1), x)
    xc = np.tile(rng.standard_normal(5), (8, 1))
    assert np.allclose(M.compress_blocks(xc, g, 4), xc[:2], atol=1e-14)


def test_compress_dominant_gate_selects_token():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((128, 32))
    g = rng.standard_normal((128, 1))
    g[3::4] += 60.0                      # the last token of every block dominates
    C = M.compress_blocks(x, g, 4)
    assert np.allclose(C, x[3::4], rtol=0, atol=1e-24 + 4 * math.exp(-55.0))


def test_compress_convex_combination_bounds():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((512, 8))
    g = rng.standard_normal((512, 8)) * 3
    for m in (4, 128):
        C = M.compress_blocks(x, g, m)
        xb = x.reshape(-1, m, 8)
        assert np.all(C <= xb.max(axis=1) + 1e-12)
        assert np.all(C >= xb.min(axis=1) - 1e-12)


def test_compress_per_channel_gate_equals_scalar_when_channels_agree():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 6))
    g = rng.standard_normal((32, 1))
    assert np.allclose(M.compress_blocks(x, g, 4), M.compress_blocks(x, np.tile(g, (1, 6)), 4),
                       atol=1e-15)


def test_classic_cache_block_counts():
    c = _gold("pages_constants.json")
    blk = c["classic_block_tokens"]
    x = np.zeros((blk["value"], 4))
    g = np.zeros((blk["value"], 1))
    assert M.compress_blocks(x, g, c["m_csa"]["value"]).shape[0] == blk["csa_entries"]
    assert M.compress_blocks(x, g, c["m_hca"]["value"]).shape[0] == blk["hca_entries"]


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_unit_rms_scale_invariance_and_gamma():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 512)) * 3
    y = M.rms_norm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(M.rms_norm(7.5 * x, eps=0.0), y, atol=1e-14)
    gam = rng.uniform(0.5, 2, 512)
    assert np.allclose(M.rms_norm(x, gam, eps=0.0), y * gam, atol=1e-14)
    # eps enters as sqrt(mean + eps)
    z = np.full((1, 4), 1e-3)
    assert np.allclose(M.rms_norm(z, eps=1e-6), z / math.sqrt(1e-6 + 1e-6), rtol=1e-14)


# ---------------------------------------------------------------- RoPE
def test_rope_complex_rotation_closed_form():
    # rotation of pair i by pos*theta_i equals multiplication by exp(i*pos*theta_i)
    D, R = 12, 8
    rng = np.random.default_rng(6)
    y = rng.standard_normal(D)
    for pos in (0, 1, 5, 4096, 1048575):
        got = M.rope_partial(y, pos, R)
        assert np.array_equal(got[: D - R], y[: D - R])
        for i in range(R // 2):
            zc = complex(y[D - R + 2 * i], y[D - R + 2 * i + 1])
            theta = 10000.0 ** (-(2.0 * i) / R)
            zr = zc * complex(math.cos(pos * theta), math.sin(pos * theta))
            assert abs(got[D - R + 2 * i] - zr.real) < 1e-9
            assert abs(got[D - R + 2 * i + 1] - zr.imag) < 1e-9
    # pair 0 turns by exactly `pos` radians, pair 1 by pos * 10000^(-2/R)
    e = np.zeros(4)
    e[2] = 1.0
    assert np.allclose(M.rope_partial(e, 1, 2)[2:], [math.cos(1.0), math.sin(1.0)], atol=1e-15)


def test_rope_norm_identity_and_relative_position():
    rng = np.random.default_rng(7)
    D, R = 512, 64
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    assert np.array_equal(M.rope_partial(q, 0, R), q)
    for p in (3, 777, 65535, 1 << 20):
        assert abs(np.linalg.norm(M.rope_partial(q, p, R)) - np.linalg.norm(q)) < 1e-10
    p, s = 1000, 371
    lhs = M.rope_partial(q, p, R) @ M.rope_partial(k, s, R)
    rhs = M.rope_partial(q, p - s, R) @ k
    assert abs(lhs - rhs) < 1e-9


def test_compress_entries_positions():
    # entry j of a run starting at pos0 is rotated at pos0 + j*m
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 8))
    g = rng.standard_normal((16, 1))
    E = M.compress_entries(x, g, 4, pos0=40, R=4)
    C = M.rms_norm(M.compress_blocks(x, g, 4))
    for j in range(4):
        assert np.allclose(E[j], M.rope_partial(C[j], 40 + 4 * j, 4), atol=1e-15)


# ---------------------------------------------------------------- indexer
def test_indexer_brute_force_and_reductions():
    rng = np.random.default_rng(9)
    H, d, N = 3, 5, 7
    q = rng.standard_normal((H, d))
    w = rng.uniform(0, 1, H)
    k = rng.standard_normal((N, d))
    got = M.indexer_scores(q, w, k)
    for s in range(N):
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for c in range(d):
                dot += q[h, c] * k[s, c]
            tot += w[h] * (dot if dot > 0 else 0.0)
        assert abs(got[s] - tot) < 1e-12
    assert np.all(got >= 0)
    one = M.indexer_scores(q[:1], np.ones(1), k)
    assert np.allclose(one, np.maximum(k @ q[0], 0), atol=1e-15)
    assert np.allclose(M.indexer_scores(2.5 * q, 3 * w, k), 7.5 * got, atol=1e-12)
    assert np.all(M.indexer_scores(q, np.zeros(H), k) == 0)


def test_visibility_rule():
    assert M.visible_entries(2047, 4) == 512          # decode at L = 2048
    assert M.visible_entries(65535, 4) == 16384
    assert M.visible_entries(262143, 128) == 2048
    assert M.visible_entries(2, 4) == 0
    assert M.visible_entries(3, 4) == 1


# ---------------------------------------------------------------- top-k
def test_top_k_against_full_sort():
    rng = np.random.default_rng(10)
    for n, k in ((100, 10), (5000, 512), (64, 64), (10, 64)):
        s = rng.standard_normal(n)
        got = M.top_k(s, k)
        want = np.sort(np.argsort(-s, kind="stable")[: min(k, n)])
        assert np.array_equal(got, want)
        assert np.all(np.diff(got) > 0)


def test_top_k_ties_lowest_index_and_rescale():
    rng = np.random.default_rng(11)
    s = rng.integers(0, 4, 1000).astype(np.float64)
    got = M.top_k(s, 300)
    # brute force: all 3s first, then 2s by index ...
    chosen = []
    for lvl in (3, 2, 1, 0):
        for i in range(1000):
            if s[i] == lvl and len(chosen) < 300:
                chosen.append(i)
    assert np.array_equal(got, np.sort(chosen))
    s2 = rng.standard_normal(777)
    assert np.array_equal(M.top_k(s2, 50), M.top_k(3.0 * s2 + 0.0, 50))
    assert np.array_equal(M.top_k(s2, 1000), np.arange(777))

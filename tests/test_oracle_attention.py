"""Pins for the oracle's sink attention and decode / prefill drivers."""
import math

import numpy as np
import torch

from oracle import method as M


def _sdpa_with_sink(qhat, ents, z, scale):
    """torch scaled_dot_product_attention (float64, CPU) with the sink as one
    extra key of zero value whose logit is forced to z_h by the additive mask."""
    H, D = qhat.shape
    n = ents.shape[0]
    q = torch.from_numpy(qhat).reshape(H, 1, D)
    K = torch.zeros(H, n + 1, D, dtype=torch.float64)
    K[:, :n] = torch.from_numpy(ents)
    V = K.clone()
    mask = torch.zeros(H, 1, n + 1, dtype=torch.float64)
    mask[:, 0, n] = torch.from_numpy(z)
    out = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=scale)
    return out.reshape(H, D).numpy()


def test_sink_attention_matches_sdpa_with_extra_key():
    rng = np.random.default_rng(0)
    for H, D, n in ((8, 128, 640), (4, 16, 3), (64, 512, 200)):
        qhat = rng.standard_normal((H, D))
        ents = rng.standard_normal((n, D))
        z = rng.standard_normal(H) * 2
        scale = 1 / math.sqrt(D)
        got = M.sink_attention(qhat, ents, z, scale)
        ref = _sdpa_with_sink(qhat, ents, z, scale)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_sink_to_minus_infinity_is_softmax_attention():
    rng = np.random.default_rng(1)
    H, D, n = 4, 32, 50
    qhat = rng.standard_normal((H, D))
    ents = rng.standard_normal((n, D))
    got = M.sink_attention(qhat, ents, np.full(H, -1e30), 0.3)
    q = torch.from_numpy(qhat).reshape(H, 1, D)
    kv = torch.from_numpy(ents).expand(H, n, D)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kv, kv, scale=0.3).reshape(H, D).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_sink_large_z_sends_weight_to_zero_with_logistic_law():
    rng = np.random.default_rng(2)
    H, D, n = 3, 16, 40
    qhat = rng.standard_normal((H, D))
    ents = rng.standard_normal((n, D))
    scale = 0.25
    l = scale * qhat @ ents.T
    lse = np.log(np.exp(l).sum(axis=1))
    for zval in (-3.0, 0.0, 5.0, 40.0):
        z = np.full(H, zval)
        o, W = M.sink_attention(qhat, ents, z, scale, return_weight=True)
        assert np.allclose(W, 1.0 / (1.0 + np.exp(zval - lse)), rtol=1e-12)
    o, W = M.sink_attention(qhat, ents, np.full(H, 200.0), scale, return_weight=True)
    assert np.all(np.abs(o) < 1e-80) and np.all(W < 1e-80)


def test_minus_infinity_sink_and_empty_set():
    """z = -inf is plain softmax attention (torch SDPA without the extra key);
    an empty attended set gives the zero vector for every z, -inf included."""
    rng = np.random.default_rng(4)
    H, D, n = 4, 32, 9
    qhat = rng.standard_normal((H, D))
    ents = rng.standard_normal((n, D))
    got = M.sink_attention(qhat, ents, np.full(H, -np.inf), 0.3)
    q = torch.from_numpy(qhat).reshape(H, 1, D)
    kv = torch.from_numpy(ents).expand(H, n, D)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kv, kv, scale=0.3).reshape(H, D).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    z = np.array([-np.inf, -1.0, 0.0, 60.0])
    o, W = M.sink_attention(qhat, np.zeros((0, D)), z, 0.3, return_weight=True)
    assert o.shape == (H, D) and np.all(o == 0.0) and np.all(W == 0.0)
    o = M.decode_one(rng.standard_normal((H, D)), 2, np.zeros((0, D)), np.zeros((0, D)), z, 0.3, 4)
    assert np.all(o == 0.0)


def test_single_entry_and_equal_logits_closed_forms():
    rng = np.random.default_rng(3)
    H, D = 5, 8
    qhat = rng.standard_normal((H, D))
    v = rng.standard_normal((1, D))
    z = rng.standard_normal(H)
    o = M.sink_attention(qhat, v, z, 0.5)
    l = 0.5 * qhat @ v[0]
    sig = 1.0 / (1.0 + np.exp(z - l))
    assert np.allclose(o, sig[:, None] * v[0][None, :], rtol=1e-13)
    # qhat = 0: every logit is 0, output = mean(V) * n / (n + e^z)
    n = 17
    V = rng.standard_normal((n, D))
    o = M.sink_attention(np.zeros((H, D)), V, z, 0.5)
    assert np.allclose(o, V.mean(0)[None, :] * (n / (n + np.exp(z)))[:, None], rtol=1e-13)


def _toy_sequence(rng, L, m, D, R, H, H_I, d_I, n_win):
    N = L // m
    ents = rng.standard_normal((N, D))
    keys = rng.standard_normal((N, d_I))
    q = rng.standard_normal((H, D))
    q_idx = rng.standard_normal((H_I, d_I))
    w = rng.uniform(0, 1, H_I)
    win = rng.standard_normal((min(n_win, L), D))
    z = rng.standard_normal(H)
    return ents, keys, q, q_idx, w, win, z


def test_csa_with_k_at_least_N_equals_hca_over_same_entries():
    rng = np.random.default_rng(4)
    L, m, D, R, H = 403, 4, 64, 16, 6
    ents, keys, q, q_idx, w, win, z = _toy_sequence(rng, L, m, D, R, H, 4, 8, 128)
    p = L - 1
    N = M.visible_entries(p, m)
    o_csa, sel, _ = M.csa_decode_one(q, p, ents, keys, q_idx, w, win, z, 0.125, m, k=N + 5, R=R)
    o_hca = M.decode_one(q, p, ents, win, z, 0.125, m, idx=None, R=R)
    assert np.array_equal(sel, np.arange(N))
    assert np.allclose(o_csa, o_hca, rtol=0, atol=0)


def test_decode_equals_dense_attention_over_gathered_rows():
    # CSA decode = SDPA(+sink) over [entries[top-k] ; window] with the rotated, normalised query
    rng = np.random.default_rng(5)
    L, m, D, R, H = 1200, 4, 32, 16, 4
    ents, keys, q, q_idx, w, win, z = _toy_sequence(rng, L, m, D, R, H, 2, 8, 128)
    p = L - 1
    o, sel, I = M.csa_decode_one(q, p, ents, keys, q_idx, w, win, z, 0.2, m, k=64, R=R)
    assert len(sel) == 64
    qn = q / np.sqrt(np.mean(q * q, axis=1, keepdims=True) + 1e-6)
    ang = p * 10000.0 ** (-np.arange(0, R, 2) / R)
    qc = qn[:, D - R::2] + 1j * qn[:, D - R + 1::2]
    qc = qc * np.exp(1j * ang)
    qhat = qn.copy()
    qhat[:, D - R::2] = qc.real
    qhat[:, D - R + 1::2] = qc.imag
    E = np.concatenate([ents[sel], win])
    assert np.allclose(o, _sdpa_with_sink(qhat, E, z, 0.2), rtol=1e-11, atol=1e-13)
    # the chosen set really holds the 64 largest scores
    thr = np.sort(I)[-64]
    assert np.all(I[sel] >= thr) and np.sum(I > thr) <= 64


def test_window_positions_rule():
    assert list(M.window_positions(5, 128)) == list(range(0, 6))
    assert list(M.window_positions(1000, 128)) == list(range(873, 1001))
    assert len(M.window_positions(65535, 128)) == 128


def test_prefill_equals_decode_with_same_window_rows():
    rng = np.random.default_rng(6)
    m, D, R, H, n_win = 4, 32, 16, 3, 16
    T0, T = 100, 60                      # token run starts at absolute position 100
    tok = rng.standard_normal((T, D))
    ents = rng.standard_normal((50, D))
    z = rng.standard_normal(H)
    for pos in (130, 159):
        q = rng.standard_normal((H, D))
        sel = np.array([0, 3, 7, 20])
        o_p = M.prefill_one(q, pos, ents, tok, T0, z, 0.3, m, n_win, idx=sel, R=R)
        win = tok[pos - n_win + 1 - T0: pos + 1 - T0]
        o_d = M.decode_one(q, pos, ents, win, z, 0.3, m, idx=sel, R=R)
        assert np.array_equal(o_p, o_d)
        # entries beyond the visible range are ignored even if listed
        o_x = M.prefill_one(q, pos, ents, tok, T0, z, 0.3, m, n_win,
                            idx=np.array([0, 3, 7, 20, M.visible_entries(pos, m)]), R=R)
        assert np.array_equal(o_x, o_p)

"""The CSA / HCA hybrid compressed attention path, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Sources (page title -- section):
  [V4blog]   "DeepSeek-V4" (haiqwa.github.io) -- CSA：压缩稀疏注意力, HCA：重度压缩注意力,
             RMSNorm归一化, Partial RoPE位置编码, 让注意力学会"忽略", FP4精度加速,
             百万 token 怎么切分到多张卡 (index visibility)
  [V4news]   硅星人 article on DeepSeek V4 -- the CSA paragraph (compressor with
             m=4, lightning indexer, ReLU multi-head index scores, top-k 512 /
             1024, 128-token window, multi-query attention), the HCA paragraph
             (m'=128, no indexer / top-k), the sink and partial-RoPE paragraph
             (last 64 dims, BF16 RoPE dims + FP8 rest), the cache paragraph
             (state cache with leftovers, classic cache blocks)
  [QbitAI]   QbitAI piece on batch invariance -- definition; no split-KV
  [V4summary] ai-engineering summary -- HCA folds 128 tokens; head_dim 512

The method is not an exact accelerator of a simpler definition (compression
and top-k change the result), so each step below is the step itself.
Readings of what the pages leave open are collected in READINGS; the GPU
library implements the same readings independently.

Pins (tests/test_oracle_method.py, tests/test_oracle_attention.py):
  compress  -- block mean for equal gates, identity for m=1, convex bounds,
               dominant-gate selection, hand-worked fixture in tests/golden
  rms_norm  -- unit RMS, scale invariance, gamma scaling
  rope      -- norm preservation, identity at position 0, relative-position
               identity, untouched non-RoPE dims, closed-form single pair
  indexer   -- brute-force loops, H_I=1 reduction to ReLU(q.k), homogeneity
  top_k     -- full sort, k >= N, positive rescale, adversarial ties
  attention -- torch scaled_dot_product_attention with the sink as an extra
               zero-value key, z -> -inf and z -> +inf limits, closed forms
               for one entry and for equal logits
  decode    -- top-k >= N reduces CSA to HCA over the same entries
  prefill   -- equals decode at the same position with the same window rows
"""

import numpy as np

READINGS = {
    "A1 compressor": "softmax over the m tokens of a block of per-token (or per-channel) "
                     "gate logits; entry = gate-weighted sum of the block's token vectors",
    "A2 leftovers": "an incomplete trailing block is not compressed (state cache holds it)",
    "A3 windows": "non-overlapping blocks of stride m",
    "A4 index keys": "one d_I key per compressed entry shared by all indexer heads; "
                     "no RMSNorm / RoPE on the indexer path",
    "A5 score": "I_s = sum_h w_h * ReLU(q_h . k_s), no scale (a positive scale keeps the ranking)",
    "A6 visibility": "query at absolute position p sees entries s < floor((p+1)/m)",
    "A7 top-k": "ties go to the lower index; N <= k keeps all; output ascending, -1 padded",
    "A8 RMSNorm": "over all D dims, eps = 1e-6, applied before RoPE",
    "A9 RoPE": "interleaved adjacent pairs (D-R+2i, D-R+2i+1), theta_i = base^(-2i/R), "
               "base 10000; entry j of a block run starting at pos0 sits at pos0 + j*m",
    "A10 cache": "E4M3 (OCP) for dims [0, D-R), BF16 for [D-R, D); no scale factors",
    "A11 K=V": "the stored entry serves as both key and value",
    "A12 scale": "softmax scale 1/sqrt(D) (an argument)",
    "A13 sink": "z_h is on the scaled-logit scale; exp(z_h) joins the denominator only",
    "A14 overlap": "window and compressed entries are both used, no de-duplication",
    "A15 window": "min(n_win, p+1) tokens ending at p inclusive",
    "A25 empty set": "a query with no compressed entry and no window row attends nothing: "
                     "its output is the empty weighted sum, 0, for every sink value",
}

ROPE_BASE = 10000.0
EPS = 1e-6


# ------------------------------------------------------------ a1: compressor
def compress_blocks(x, gate, m):
    """Softmax-gated block sum ([V4news] CSA/HCA paragraphs: every m tokens'
    KV fold into one entry; the gate convention is reading A1).

    x    : [T, D] token vectors, T % m == 0
    gate : [T, 1] (one logit per token) or [T, D] (one per channel)
    returns C : [T // m, D]
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    T, D = x.shape
    assert T % m == 0
    nb = T // m
    xb = x.reshape(nb, m, D)
    gb = g.reshape(nb, m, g.shape[1])
    gmax = gb.max(axis=1, keepdims=True)
    e = np.exp(gb - gmax)
    w = e / e.sum(axis=1, keepdims=True)        # softmax over the block's tokens
    return (w * xb).sum(axis=1)                 # broadcasts a [.., 1] gate over D


# ------------------------------------------------------------ a4: norm + RoPE
def rms_norm(x, gamma=None, eps=EPS):
    """RMSNorm over the last axis ([V4blog] RMSNorm归一化: applied to every query
    head and to the single compressed KV head before core attention)."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rope_angles(pos, R, base=ROPE_BASE):
    """pos * base^(-2i/R) for i < R/2; pos is an int array."""
    i = np.arange(R // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / R)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rope_partial(y, pos, R, base=ROPE_BASE):
    """Rotate the last R dims of y ([V4blog] Partial RoPE; [V4news]: RoPE on the
    last 64 dims of queries and KV only).  Pairs are (D-R+2i, D-R+2i+1) and
    pair i turns by pos * base^(-2i/R) (reading A9).

    y   : [..., D]; pos broadcastable to y.shape[:-1]
    """
    y = np.array(y, dtype=np.float64, copy=True)
    if R == 0:
        return y
    D = y.shape[-1]
    ang = rope_angles(np.broadcast_to(np.asarray(pos), y.shape[:-1]), R, base)
    c, s = np.cos(ang), np.sin(ang)
    a = y[..., D - R::2].copy()
    b = y[..., D - R + 1::2].copy()
    y[..., D - R::2] = a * c - b * s
    y[..., D - R + 1::2] = a * s + b * c
    return y


def compress_entries(x, gate, m, pos0, norm_w=None, eps=EPS, R=0, base=ROPE_BASE,
                     normalize=True):
    """Full write path of one run of tokens starting at absolute position pos0:
    block sum -> RMSNorm -> partial RoPE at the block's first position.
    Returns float64 entries before quantisation to the cache format."""
    C = compress_blocks(x, gate, m)
    if normalize:
        C = rms_norm(C, norm_w, eps)
    pos = pos0 + m * np.arange(C.shape[0])
    return rope_partial(C, pos, R, base)


# ------------------------------------------------------------ a2: indexer
def indexer_scores(q_idx, w, keys):
    """Lightning-indexer scores ([V4news] CSA paragraph and indexer detail:
    multi-head index queries, ReLU, scores against compressed index keys).

    q_idx : [H_I, d_I], w : [H_I], keys : [N, d_I]  ->  I : [N]
    I_s = sum_h w_h * max(0, q_h . k_s)      (reading A5)
    """
    dots = np.asarray(keys, np.float64) @ np.asarray(q_idx, np.float64).T   # [N, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


def visible_entries(p, m):
    """Entries visible to a query at absolute position p (reading A6; [V4blog]
    index visibility is a precomputable rule)."""
    return (p + 1) // m


# ------------------------------------------------------------ a3: top-k
def top_k(scores, k):
    """The k best entries ([V4news]: the top-k selector keeps the 512 (Pro:
    1024) most relevant compressed blocks).  Order by score descending, then
    index ascending; return the chosen indices ascending (reading A7)."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))      # primary: -s, secondary: index
    chosen = order[: min(k, n)]
    return np.sort(chosen)


# ------------------------------------------------------------ a5: sink MQA
def sink_attention(qhat, ents, z, scale, return_weight=False):
    """Single-KV-head attention with a per-head sink logit.

    [V4news]: selected entries plus the window go to core multi-query
    attention; each head has a learnable sink logit added to the softmax
    denominator.  [V4blog] 让注意力学会"忽略": a large z'_h shrinks every weight.
    K = V = the stored entry (A11); z on the scaled-logit scale (A13).

    qhat : [H, D] (already normalised and rotated), ents : [n, D], z : [H]
    o_h = sum_j e^{l_hj} v_j / (sum_j e^{l_hj} + e^{z_h}),  l = scale * qhat . ents^T
    """
    qhat = np.asarray(qhat, np.float64)
    ents = np.asarray(ents, np.float64)
    z = np.asarray(z, np.float64)
    if ents.shape[0] == 0:
        # nothing attended: the numerator is an empty sum, so the output is 0
        # whatever the sink (for z = -inf the denominator is empty too)
        o = np.zeros((qhat.shape[0], ents.shape[1] if ents.ndim == 2 else qhat.shape[1]))
        return (o, np.zeros(qhat.shape[0])) if return_weight else o
    logits = scale * (qhat @ ents.T)                              # [H, n]
    M = np.maximum(z, logits.max(axis=1) if ents.shape[0] else -np.inf)
    e = np.exp(logits - M[:, None])
    den = e.sum(axis=1) + np.exp(z - M)
    o = (e @ ents) / den[:, None]
    if return_weight:
        return o, 1.0 - np.exp(z - M) / den
    return o


def query_prologue(q, pos, norm_w=None, eps=EPS, R=0, base=ROPE_BASE):
    """RMSNorm of every query head, then partial RoPE at the query position."""
    return rope_partial(rms_norm(q, norm_w, eps), pos, R, base)


def decode_one(q, pos, ents, win_ents, z, scale, m, idx=None, norm_w=None, eps=EPS,
               R=0, base=ROPE_BASE, return_weight=False):
    """One decode query.

    q        : [H, D] raw query heads
    pos      : absolute position p of the query
    ents     : [>= N, D] this sequence's compressed entries (decoded values)
    win_ents : [w, D] window rows, oldest first, the last at position p
    idx      : ascending selected entry indices (CSA, may contain -1 padding)
               or None (HCA: all N visible entries)
    """
    N = visible_entries(pos, m)
    if idx is None:
        sel = np.arange(N)
    else:
        idx = np.asarray(idx)
        sel = idx[(idx >= 0) & (idx < N)]
    E = np.concatenate([np.asarray(ents, np.float64)[sel],
                        np.asarray(win_ents, np.float64)], axis=0)
    qhat = query_prologue(q, pos, norm_w, eps, R, base)
    return sink_attention(qhat, E, z, scale, return_weight)


def window_positions(p, n_win):
    """Positions of the sliding window of a query at p (reading A15)."""
    return np.arange(max(0, p - n_win + 1), p + 1)


def csa_decode_one(q, pos, ents, keys, q_idx, w, win_ents, z, scale, m, k, **kw):
    """Indexer -> top-k -> sink MQA for one decode query (the CSA layer)."""
    N = visible_entries(pos, m)
    I = indexer_scores(q_idx, w, np.asarray(keys)[:N])
    sel = top_k(I, k)
    return decode_one(q, pos, ents, win_ents, z, scale, m, idx=sel, **kw), sel, I


def prefill_one(q, pos, ents, tok_rows, tok_pos0, z, scale, m, n_win, idx=None, **kw):
    """One causal prefill query at absolute position pos.

    tok_rows : [T, D] normalised, rotated per-token rows of a run whose first
               row sits at absolute position tok_pos0; the query's window is
               the rows at positions max(0, pos-n_win+1) .. pos (A15).
    idx      : its own ascending top-k entry indices (CSA) or None (HCA).
    Decode and prefill of the same token see the same entries, so this is
    decode_one with the window cut out of the token run.
    """
    wp = window_positions(pos, n_win)
    assert wp[0] >= tok_pos0, "token run must cover the whole window"
    win = np.asarray(tok_rows, np.float64)[wp - tok_pos0]
    return decode_one(q, pos, ents, win, z, scale, m, idx=idx, **kw)

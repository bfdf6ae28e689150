"""Seeded synthetic inputs for the CSA / HCA path.

This module only draws random numbers and lays them out in the byte formats
the library reads.  It holds none of the method's arithmetic: no compression,
normalisation, rotation, scoring, selection or attention.  Storage casts to
bfloat16 and FP8-E4M3 use torch's dtype conversions (round to nearest even);
MXFP4 rows are drawn directly as random E2M1 codes and E8M0 scale bytes.

Workloads (WORKLOADS, keyed by name):
  * csa_decode_fp32_b1_ctx2048 -- CSA decode, fp32, 1 sequence of 2048 tokens,
            D=128, 8 heads, indexer 4 x 64, top-k 64, window 128;
  * csa_decode_b16_ctx65536 -- CSA decode, 16 sequences of 65,536 tokens
            (16,384 entries), D=512 split cache, 64 heads, FP8 indexer
            64 x 128, top-k 512;
  * hca_decode_b32_ctx262144 -- HCA decode, 32 sequences of 262,144 tokens,
            m'=128 (2048 entries);
  * csa_prefill_ctx131072_chunk2048 -- CSA prefill chunk: 131,072 cached +
            2048 new tokens, top-k 1024;
  * ragged_csa_hca_b64_ctx1k_1m -- ragged CSA (MXFP4 indexer, top-k 1024) +
            HCA decode, 64 sequences with lengths log-uniform in [1024, 1048576].
Hidden values are N(0,1) before quantisation; indexer head weights U(0,1);
sink logits N(0,1).
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

F32, BF16, FP8, MXFP4, SPLIT = 0, 1, 2, 3, 4


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(seed))


def row_bytes(fmt, D, R=0):
    return {F32: 4 * D, BF16: 2 * D, FP8: D, MXFP4: D // 2 + D // 32,
            SPLIT: (D - R) + 2 * R}[fmt]


def _bf16_bytes(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint8).reshape(x32.shape[:-1] + (-1,))


def _fp8_bytes(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().reshape(x32.shape)


def random_rows(rng, n, D, fmt, R=0, chunk=1 << 16, mx_scales=(124, 128)):
    """n rows of N(0,1) values stored in `fmt`; uint8 [n, row_bytes].  MXFP4
    rows hold uniform random E2M1 codes and E8M0 scale bytes drawn uniformly
    from [mx_scales[0], mx_scales[1])."""
    rb = row_bytes(fmt, D, R)
    out = np.empty((n, rb), dtype=np.uint8)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        if fmt == MXFP4:
            codes = rng.integers(0, 16, size=(b - a, D), dtype=np.uint8)
            out[a:b, : D // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
            out[a:b, D // 2:] = rng.integers(mx_scales[0], mx_scales[1], size=(b - a, D // 32), dtype=np.uint8)
            continue
        x = rng.standard_normal((b - a, D), dtype=np.float32)
        if fmt == F32:
            out[a:b] = x.view(np.uint8).reshape(b - a, rb)
        elif fmt == BF16:
            out[a:b] = _bf16_bytes(x)
        elif fmt == FP8:
            out[a:b] = _fp8_bytes(x)
        elif fmt == SPLIT:
            out[a:b, : D - R] = _fp8_bytes(x[:, : D - R])
            out[a:b, D - R:] = _bf16_bytes(x[:, D - R:])
        else:
            raise ValueError(fmt)
    return out


def log_uniform_lengths(rng, n, lo, hi):
    return np.round(np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))).astype(np.int64)


@dataclass
class DecodeInputs:
    """One batch of decode queries over ragged per-sequence caches."""
    B: int
    H: int
    D: int
    R: int
    m: int
    n_win: int
    lengths: np.ndarray            # [B] context length including the new token
    q_pos: np.ndarray              # [B] int64 = lengths - 1
    kv_fmt: int
    kv: np.ndarray                 # uint8 [sum N, row_bytes]
    kv_off: np.ndarray             # [B] int64 first row of each sequence
    n_ent: np.ndarray              # [B] entries in each sequence's cache
    q_fmt: int
    q: np.ndarray                  # uint8 [B, H, row_bytes]
    win_fmt: int
    win: np.ndarray                # uint8 [B, n_win, row_bytes]
    win_len: np.ndarray            # [B] int32
    sinks: np.ndarray              # [H] float32
    scale: float
    # indexer part (CSA only)
    k: int = 0
    idx_fmt: int = FP8
    H_I: int = 0
    d_I: int = 0
    keys: Optional[np.ndarray] = None    # uint8 [sum N, row_bytes]
    q_idx: Optional[np.ndarray] = None   # uint8 [B, H_I, row_bytes]
    w: Optional[np.ndarray] = None       # float32 [B, H_I]
    extra: dict = field(default_factory=dict)


def decode_inputs(seed, lengths, *, m, H, D, R, n_win=128, kv_fmt=SPLIT, q_fmt=BF16,
                  win_fmt=BF16, csa=True, k=512, idx_fmt=FP8, H_I=64, d_I=128, rng=None,
                  mx_scales=(124, 128)):
    """Seeded decode batch.  Draw order: lengths (given) -> cache entries ->
    window rows -> queries -> index keys -> index queries -> head weights ->
    sinks.  mx_scales: range of the E8M0 scale bytes of MXFP4 index rows."""
    rng = rng or rng_for(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = lengths.shape[0]
    n_ent = lengths // m
    kv_off = np.zeros(B, dtype=np.int64)
    kv_off[1:] = np.cumsum(n_ent)[:-1]
    kv = random_rows(rng, int(n_ent.sum()), D, kv_fmt, R)
    win = random_rows(rng, B * n_win, D, win_fmt, R).reshape(B, n_win, row_bytes(win_fmt, D, R))
    win_len = np.minimum(n_win, lengths).astype(np.int32)
    q = random_rows(rng, B * H, D, q_fmt, R).reshape(B, H, row_bytes(q_fmt, D, R))
    keys = q_idx = w = None
    if csa:
        keys = random_rows(rng, int(n_ent.sum()), d_I, idx_fmt, mx_scales=mx_scales)
        q_idx = random_rows(rng, B * H_I, d_I, idx_fmt, mx_scales=mx_scales).reshape(B, H_I, row_bytes(idx_fmt, d_I))
        w = rng.uniform(0.0, 1.0, size=(B, H_I)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    return DecodeInputs(B=B, H=H, D=D, R=R, m=m, n_win=n_win, lengths=lengths,
                        q_pos=lengths - 1, kv_fmt=kv_fmt, kv=kv, kv_off=kv_off, n_ent=n_ent,
                        q_fmt=q_fmt, q=q, win_fmt=win_fmt, win=win, win_len=win_len,
                        sinks=sinks, scale=float(1.0 / np.sqrt(D)), k=k, idx_fmt=idx_fmt,
                        H_I=H_I, d_I=d_I, keys=keys, q_idx=q_idx, w=w)


@dataclass
class TokenInputs:
    """Raw per-token vectors and gate logits for the compressor."""
    x: np.ndarray          # float32 [T, D]
    gate: np.ndarray       # float32 [T, gate_cols]


def token_inputs(seed, T, D, gate_cols=1, rng=None):
    rng = rng or rng_for(seed)
    x = rng.standard_normal((T, D), dtype=np.float32)
    g = rng.standard_normal((T, gate_cols), dtype=np.float32)
    return TokenInputs(x=x, gate=g)


def random_scores(seed, nq, ld, n_valid=None, tie_levels=0, rng=None):
    """Score rows for the top-k selector.  tie_levels > 0 draws integers in
    [0, tie_levels) (many exact ties); otherwise N(0,1) float32."""
    rng = rng or rng_for(seed)
    if tie_levels:
        s = rng.integers(0, tie_levels, size=(nq, ld)).astype(np.float32)
    else:
        s = rng.standard_normal((nq, ld), dtype=np.float32)
    if n_valid is None:
        n_valid = np.full(nq, ld, dtype=np.int64)
    return s, np.asarray(n_valid, dtype=np.int64)


# --------------------------------------------------------------- workloads
WORKLOADS = {
    "csa_decode_fp32_b1_ctx2048": dict(seed=1, B=1, L=2048, m=4, H=8, D=128, R=64,
            n_win=128, k=64, H_I=4, d_I=64, kv_fmt=F32, q_fmt=F32, win_fmt=F32,
            idx_fmt=F32, csa=True),
    "csa_decode_b16_ctx65536": dict(seed=2, B=16, L=65536, m=4, H=64, D=512, R=64,
            n_win=128, k=512, H_I=64, d_I=128, kv_fmt=SPLIT, q_fmt=BF16, win_fmt=BF16,
            idx_fmt=FP8, csa=True),
    "hca_decode_b32_ctx262144": dict(seed=3, B=32, L=262144, m=128, H=64, D=512, R=64,
            n_win=128, kv_fmt=SPLIT, q_fmt=BF16, win_fmt=BF16, csa=False),
    "csa_prefill_ctx131072_chunk2048": dict(seed=4, cached=131072, chunk=2048, m=4, H=64,
            D=512, R=64, n_win=128, k=1024, H_I=64, d_I=128, kv_fmt=SPLIT, q_fmt=BF16,
            idx_fmt=FP8),
    "ragged_csa_hca_b64_ctx1k_1m": dict(seed=5, B=64, Lmin=1024, Lmax=1048576, m=4, m_hca=128,
            H=64, D=512, R=64, n_win=128, k=1024, H_I=64, d_I=128, kv_fmt=SPLIT,
            q_fmt=BF16, win_fmt=BF16, idx_fmt=MXFP4),
}


def workload_decode_inputs(name, seed=None, B=None, L=None):
    """Decode inputs of a decode workload (optionally with a smaller B or L)."""
    c = WORKLOADS[name]
    seed = c["seed"] if seed is None else seed
    B = c["B"] if B is None else B
    L = c["L"] if L is None else L
    lengths = np.full(B, L, dtype=np.int64)
    return decode_inputs(seed, lengths, m=c["m"], H=c["H"], D=c["D"], R=c["R"],
                         n_win=c["n_win"], kv_fmt=c["kv_fmt"], q_fmt=c["q_fmt"],
                         win_fmt=c["win_fmt"], csa=c["csa"], k=c.get("k", 0),
                         idx_fmt=c.get("idx_fmt", FP8), H_I=c.get("H_I", 0),
                         d_I=c.get("d_I", 0))


def random_selection(rng, n_ent, k):
    """Per row: an ascending random subset of min(k, N) entry indices, -1 padded
    (a stand-in for a top-k result when only the attention is under test)."""
    n_ent = np.asarray(n_ent)
    out = np.full((n_ent.shape[0], k), -1, dtype=np.int32)
    for b, N in enumerate(n_ent):
        c = min(k, int(N))
        if c:
            out[b, :c] = np.sort(rng.choice(int(N), size=c, replace=False)).astype(np.int32)
    return out


# --------------------------------------------------------------- device-side generation
# Full-size inputs (hundreds of MB) are drawn on the GPU with a seeded torch
# generator; tests copy back only the rows the oracle needs.  Same value
# distributions as the host generators above.
def device_generator(seed, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def device_rows(gen, n, D, fmt, R=0, device="cuda", chunk=1 << 16):
    """n rows of N(0,1) values stored in `fmt` on `device`; uint8 [n, row_bytes]."""
    rb = row_bytes(fmt, D, R)
    out = torch.empty((n, rb), dtype=torch.uint8, device=device)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        if fmt == MXFP4:
            codes = torch.randint(0, 16, (b - a, D), generator=gen, device=device, dtype=torch.uint8)
            out[a:b, : D // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
            out[a:b, D // 2:] = torch.randint(124, 128, (b - a, D // 32), generator=gen, device=device,
                                              dtype=torch.uint8)
            continue
        x = torch.randn((b - a, D), generator=gen, device=device, dtype=torch.float32)
        if fmt == F32:
            out[a:b] = x.view(torch.uint8).reshape(b - a, rb)
        elif fmt == BF16:
            out[a:b] = x.to(torch.bfloat16).view(torch.uint8).reshape(b - a, rb)
        elif fmt == FP8:
            out[a:b] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        elif fmt == SPLIT:
            out[a:b, : D - R] = x[:, : D - R].to(torch.float8_e4m3fn).view(torch.uint8)
            out[a:b, D - R:] = x[:, D - R:].contiguous().to(torch.bfloat16).view(torch.uint8).reshape(b - a, 2 * R)
        else:
            raise ValueError(fmt)
    return out


def device_decode_inputs(seed, lengths, *, m, H, D, R, n_win=128, csa=True, k=512, idx_fmt=FP8,
                         H_I=64, d_I=128, device="cuda"):
    """A decode batch like decode_inputs, drawn on the device (same draw
    order; returns device tensors plus host metadata in a dict)."""
    gen = device_generator(seed, device)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = lengths.shape[0]
    n_ent = lengths // m
    kv_off = np.zeros(B, dtype=np.int64)
    kv_off[1:] = np.cumsum(n_ent)[:-1]
    d = dict(B=B, H=H, D=D, R=R, m=m, n_win=n_win, k=k, idx_fmt=idx_fmt, H_I=H_I, d_I=d_I,
             lengths=lengths, n_ent=n_ent, kv_off=kv_off, q_pos=lengths - 1,
             win_len=np.minimum(n_win, lengths).astype(np.int32), scale=float(1.0 / np.sqrt(D)))
    d["kv"] = device_rows(gen, int(n_ent.sum()), D, SPLIT, R, device)
    d["win"] = device_rows(gen, B * n_win, D, BF16, R, device).reshape(B, n_win, -1)
    d["q"] = device_rows(gen, B * H, D, BF16, R, device).reshape(B, H, -1)
    if csa:
        d["keys"] = device_rows(gen, int(n_ent.sum()), d_I, idx_fmt, 0, device)
        d["q_idx"] = device_rows(gen, B * H_I, d_I, idx_fmt, 0, device).reshape(B, H_I, -1)
        d["w"] = torch.rand((B, H_I), generator=gen, device=device, dtype=torch.float32)
    d["sinks"] = torch.randn(H, generator=gen, device=device, dtype=torch.float32)
    return d

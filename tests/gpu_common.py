"""Shared helpers of the GPU parity tests: upload seeded inputs, run the
library through its C ABI, and compute the oracle's answer from the same
bytes (decoded by the oracle's own format code)."""
import numpy as np
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from oracle import formats as OF
from oracle import method as OM

DEV = "cuda:0"
EPS = 1e-6
ROPE_BASE = 10000.0


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def gpu_bytes(n):
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def run_decode(inp, idx_t=None, variant=csa.VARIANT_AUTO, bufs=None):
    """hybrid_attn_decode on a synth.DecodeInputs; returns the raw output bytes (uint8 [B,H,rb])."""
    B, H, D, R = inp.B, inp.H, inp.D, inp.R
    if bufs is None:
        bufs = upload_decode(inp)
    out_fmt = csa.F32 if inp.q_fmt == csa.F32 else csa.BF16
    out = gpu_bytes(B * H * csa.row_bytes(out_fmt, D))
    csa.hybrid_attn_decode(bufs["q"], inp.q_fmt, B, H, D, bufs["q_pos"], None, EPS, R, ROPE_BASE,
                           bufs["kv"], inp.kv_fmt, bufs["kv_off"], inp.m, idx_t,
                           inp.k if idx_t is not None else 0, bufs["win"], inp.win_fmt, inp.n_win,
                           bufs["win_len"], bufs["sinks"], inp.scale, out, out_fmt, variant)
    return out, bufs


def upload_decode(inp):
    b = dict(q=dev(inp.q), q_pos=dev(inp.q_pos), kv=dev(inp.kv), kv_off=dev(inp.kv_off),
             win=dev(inp.win), win_len=dev(inp.win_len), sinks=dev(inp.sinks))
    if inp.keys is not None:
        b.update(keys=dev(inp.keys), q_idx=dev(inp.q_idx), w=dev(inp.w))
    return b


def decode_out(out, fmt, B, H, D):
    raw = out.cpu().numpy()
    return OF.decode_rows(raw, fmt, D).reshape(B, H, D)


def oracle_decode_query(inp, b, sel=None):
    """Oracle output [H, D] of query b; sel = ascending selected indices or None (HCA)."""
    D, R = inp.D, inp.R
    rb = synth.row_bytes(inp.kv_fmt, D, R)
    N = int(inp.n_ent[b])
    p = int(inp.q_pos[b])
    kv_rows = inp.kv[int(inp.kv_off[b]): int(inp.kv_off[b]) + N]
    ents = OF.decode_rows(kv_rows, inp.kv_fmt, D, R) if N else np.zeros((0, D))
    wl = int(inp.win_len[b])
    win = OF.decode_rows(inp.win[b, :wl], inp.win_fmt, D, R) if wl else np.zeros((0, D))
    q = OF.decode_rows(inp.q[b], inp.q_fmt, D, R)
    return OM.decode_one(q, p, ents, win, inp.sinks.astype(np.float64), inp.scale, inp.m,
                         idx=sel, eps=EPS, R=R, base=ROPE_BASE)


def oracle_scores(inp, b):
    N = int(inp.n_ent[b])
    keys = OF.decode_rows(inp.keys[int(inp.kv_off[b]): int(inp.kv_off[b]) + N], inp.idx_fmt, inp.d_I)
    qi = OF.decode_rows(inp.q_idx[b], inp.idx_fmt, inp.d_I)
    return OM.indexer_scores(qi, inp.w[b].astype(np.float64), keys)


def assert_lowp_close(got, ref, tol=2e-2, what=""):
    """Low-precision bar: per (query, head), max |gpu - oracle| <= tol * rms(oracle).
    The whole difference counts, the rounding of the BF16 output included."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    err = np.abs(got - ref) / rms
    worst = float(err.max())
    assert worst <= tol, f"{what}: max |gpu - oracle| / rms(oracle) = {worst:.3g} > {tol}"
    return worst


def assert_f32_close(got, ref, tol=1e-5, what=""):
    """fp32 bar: per (query, head) ||gpu - oracle||_inf <= tol * ||oracle||_inf."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    worst = float((num / den).max())
    assert worst <= tol, f"{what}: normwise relative error {worst:.3g} > {tol}"
    return worst

"""Number formats used by the cache and the indexer, written from their specs.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Where the pages fix the precision:
  * the KV cache keeps the 64 RoPE dims in BF16 and the other dims in FP8
    (DeepSeek-V4 blog, section "Partial RoPE"; 硅星人 article, paragraph on the
    RoPE-dims / mixed-precision cache);
  * the lightning indexer runs at FP4 (DeepSeek-V4 blog, section "FP4精度加速").
The pages do not define the formats themselves; this module follows
  * bfloat16: IEEE-754 binary32 with the low 16 bits dropped, round to nearest
    even;
  * FP8 E4M3 as in the OCP 8-bit floating point spec (bias 7, no infinities,
    S.1111.111 is NaN, max normal 448, subnormals m * 2^-9);
  * E2M1 elements and E8M0 scales as in the OCP Microscaling (MX) spec v1.0
    (32-element blocks, shared scale 2^(floor(log2 amax) - 2));
  * the "split" cache row: (D-R) E4M3 bytes, then R little-endian bfloat16.

All rounding is done on exact float64 values with numpy.rint (round half to
even) on a binary grid, so nothing here depends on float32 arithmetic.
Pins (tests/test_oracle_formats.py): exhaustive comparison of every FP8 code
with torch.float8_e4m3fn, BF16 rounding against torch.bfloat16, the E2M1 value
table from tests/golden, tie-to-even and saturation cases, and MXFP4 grid
round trips.
"""

import numpy as np

# Format identifiers; the C header uses the same numbering.
F32, BF16, FP8, MXFP4, SPLIT = 0, 1, 2, 3, 4


def _round_to_grid(x, mant_bits, emin, max_finite, saturate):
    """Round float64 `x` to a binary float grid with `mant_bits` fraction bits,
    minimum normal exponent `emin` (subnormals below it) and largest finite
    magnitude `max_finite`, round half to even.  Overflow saturates to
    +-max_finite when `saturate`, else becomes +-inf.  NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x)
    ax = np.abs(np.where(fin, x, 0.0))
    nz = ax > 0
    # exponent of the leading bit, floor(log2 |x|), exact via frexp
    _, e = np.frexp(np.where(nz, ax, 1.0))
    e = e.astype(np.int64) - 1
    e = np.maximum(e, emin)              # subnormal range shares emin's spacing
    ulp = np.ldexp(1.0, (e - mant_bits).astype(np.int64))
    q = np.rint(ax / ulp) * ulp          # rint = round half to even
    over = q > max_finite
    if saturate:
        q = np.where(over, max_finite, q)
    else:
        q = np.where(over, np.inf, q)
    out = np.where(fin, np.copysign(q, x), x)
    if not saturate:
        out = np.where(np.isinf(x), x, out)
    else:
        out = np.where(np.isinf(x), np.copysign(max_finite, x), out)
    return out


# ---------------------------------------------------------------- bfloat16
def bf16_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x):
    """Nearest bfloat16 value (as float64), ties to even, overflow to inf."""
    return _round_to_grid(x, 7, -126, float(np.float32(3.3895313892515355e38)), False)


def f64_to_bf16_bits(x):
    v = round_bf16(x).astype(np.float32)   # exact: every bf16 value is an f32
    return (v.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- FP8 E4M3
def e4m3_to_f64(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = s * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


E4M3_MAX = 448.0


def round_e4m3(x):
    """Nearest E4M3 value, ties to even, saturating at +-448."""
    return _round_to_grid(x, 3, -6, E4M3_MAX, True)


_E4M3_POS = e4m3_to_f64(np.arange(128, dtype=np.uint8))  # codes 0..127


def f64_to_e4m3_bits(x):
    x = np.asarray(x, dtype=np.float64)
    v = round_e4m3(x)
    out = np.zeros(v.shape, dtype=np.uint8)
    nan = np.isnan(v)
    av = np.abs(np.where(nan, 0.0, v))
    # positive codes 0..126 are strictly increasing in value
    idx = np.searchsorted(_E4M3_POS[:127], av)
    out = idx.astype(np.uint8) | np.where(np.signbit(v) & ~nan, 0x80, 0).astype(np.uint8)
    out = np.where(nan, np.uint8(0x7F), out)
    return out.astype(np.uint8)


# ---------------------------------------------------------------- E2M1 / E8M0
def e2m1_to_f64(codes):
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return s * mag


E2M1_MAX = 6.0
_E2M1_POS = e2m1_to_f64(np.arange(8))


def round_e2m1(x):
    """Nearest E2M1 value, ties to even, saturating at +-6."""
    return _round_to_grid(x, 1, 0, E2M1_MAX, True)


def f64_to_e2m1_codes(x):
    v = round_e2m1(x)
    idx = np.searchsorted(_E2M1_POS, np.abs(v))
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def e8m0_to_f64(b):
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


MX_BLOCK = 32


def mxfp4_encode(x):
    """OCP MX v1.0 MXFP4 encoding of rows x[..., d] (d % 32 == 0).

    Per 32-element block: shared exponent floor(log2 amax) - 2 (2 = exponent
    of E2M1's largest normal), clamped to the E8M0 range; each element is
    x / 2^shared rounded to E2M1 (ties to even, saturating).  An all-zero block
    gets scale byte 0 and zero elements.
    Row layout: d/2 bytes of codes (element 2i in the low nibble, 2i+1 in the
    high nibble), then d/32 scale bytes.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    lead = x.shape[:-1]
    blk = x.reshape(lead + (d // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = e.astype(np.int64) - 1 - 2
    shared = np.clip(shared, -127, 127)
    sbyte = np.where(amax > 0, shared + 127, 0).astype(np.uint8)
    scale = np.ldexp(1.0, np.where(amax > 0, shared, 0))
    codes = f64_to_e2m1_codes(blk / scale[..., None])
    codes = np.where((amax > 0)[..., None], codes, 0).astype(np.uint8)
    codes = codes.reshape(lead + (d,))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, sbyte], axis=-1)


def mxfp4_decode(rows, d):
    rows = np.asarray(rows, dtype=np.uint8)
    packed = rows[..., : d // 2]
    sbyte = rows[..., d // 2: d // 2 + d // MX_BLOCK]
    codes = np.empty(rows.shape[:-1] + (d,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    vals = e2m1_to_f64(codes).reshape(rows.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    vals = vals * e8m0_to_f64(sbyte)[..., None]
    return vals.reshape(rows.shape[:-1] + (d,))


# ---------------------------------------------------------------- split rows
def split_row_bytes(D, R):
    return (D - R) + 2 * R


def split_encode(x, R):
    """Cache row: dims [0, D-R) as E4M3 codes, dims [D-R, D) as bfloat16."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    lo = f64_to_e4m3_bits(x[..., : D - R])
    hi = f64_to_bf16_bits(x[..., D - R:]).view(np.uint8)
    hi = hi.reshape(x.shape[:-1] + (2 * R,))
    return np.concatenate([lo, hi], axis=-1)


def split_decode(rows, D, R):
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8))
    lo = e4m3_to_f64(rows[..., : D - R])
    hi = bf16_to_f64(rows[..., D - R: D - R + 2 * R].copy().view(np.uint16))
    return np.concatenate([lo, hi], axis=-1)


def row_bytes(fmt, D, R=0):
    return {F32: 4 * D, BF16: 2 * D, FP8: D, MXFP4: D // 2 + D // MX_BLOCK,
            SPLIT: split_row_bytes(D, R)}[fmt]


def decode_rows(buf, fmt, D, R=0):
    """Decode a uint8 buffer of rows in format `fmt` to float64 [n, D]."""
    buf = np.ascontiguousarray(np.asarray(buf)).view(np.uint8)
    rb = row_bytes(fmt, D, R)
    rows = buf.reshape(-1, rb)
    if fmt == F32:
        return rows.copy().view(np.float32).astype(np.float64)
    if fmt == BF16:
        return bf16_to_f64(rows.copy().view(np.uint16))
    if fmt == FP8:
        return e4m3_to_f64(rows)
    if fmt == MXFP4:
        return mxfp4_decode(rows, D)
    if fmt == SPLIT:
        return split_decode(rows, D, R)
    raise ValueError(fmt)


def encode_rows(x, fmt, R=0):
    """Encode float64 rows to the byte layout of `fmt` (uint8 [n, row_bytes])."""
    x = np.asarray(x, dtype=np.float64)
    if fmt == F32:
        return x.astype(np.float32).view(np.uint8).reshape(x.shape[0], -1)
    if fmt == BF16:
        return f64_to_bf16_bits(x).view(np.uint8).reshape(x.shape[0], -1)
    if fmt == FP8:
        return f64_to_e4m3_bits(x)
    if fmt == MXFP4:
        return mxfp4_encode(x)
    if fmt == SPLIT:
        return split_encode(x, R)
    raise ValueError(fmt)

"""Exact number-format codecs for the oracle (float64 results).

The pages say that most KV entries are stored in FP8 with the RoPE
dimensions in BF16, and that the CSA lightning indexer runs in FP4
(pogovet.com, 상세 정리 §5).  They do not define the formats; the readings
taken here are the public ones:

* bfloat16: the top 16 bits of an IEEE binary32.
* fp8 e4m3: OCP 8-bit floating point, E4M3 variant (bias 7, no infinities,
  S.1111.111 is NaN, largest finite 448).
* MXFP4: OCP Microscaling v1.0 — blocks of 32 FP4 (E2M1) elements sharing one
  E8M0 scale.  Shared exponent X = floor(log2(max|v|)) - 2 (2 is the
  largest E2M1 exponent), clamped to [-127, 127]; an all-zero block takes
  X = 0.  Elements are v / 2^X rounded to nearest-even on the E2M1 grid,
  saturating to +-6.  Two elements per byte, the even element in the low
  nibble; the scale byte is X + 127.

Encoders take float32 input and make their rounding decisions on the exact
value of that float32 (float64 arithmetic on it is exact here), so that a
quantiser fed the same float32 bits must produce the same bytes.
"""
from __future__ import annotations

import numpy as np

F32, BF16, FP8_E4M3, MXFP4 = "f32", "bf16", "fp8_e4m3", "mxfp4"

# E2M1 magnitudes by 3-bit code (exponent bias 1, one mantissa bit, code 0/1 subnormal)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ----------------------------------------------------------------- bfloat16
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    f = np.asarray(x, dtype=np.float64)
    out = np.zeros(f.shape, dtype=np.uint16)
    sign = np.signbit(f)
    a = np.abs(f)
    nz = (a > 0) & np.isfinite(a)
    # bf16 normal: 8 significant bits; quantum 2^(e-7) with e = floor(log2 a), floored at -126
    e = np.zeros(f.shape, dtype=np.int64)
    mant, ex = np.frexp(a[nz])          # a = mant * 2^ex, mant in [0.5, 1)
    e[nz] = np.maximum(ex - 1, -126)
    q = np.zeros(f.shape, dtype=np.float64)
    q[nz] = np.rint(np.ldexp(a[nz], -(e[nz] - 7)))   # integer significand, ties to even
    val = np.ldexp(q, e - 7)
    out_f32 = val.astype(np.float32)
    bits = out_f32.view(np.uint32) >> np.uint32(16)
    out[:] = bits.astype(np.uint16)
    out[np.isnan(f)] = 0x7FC0
    out[np.isinf(f)] = 0x7F80
    out[sign] |= np.uint16(0x8000)
    return out


# ----------------------------------------------------------------- fp8 e4m3 (OCP)
def decode_e4m3(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = s * val
    return np.where((e == 15) & (m == 7), np.nan, val)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3 code, nearest-even, saturating to +-448, NaN -> 0x7F."""
    f = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(f)
    a = np.minimum(np.abs(f), 448.0)
    code = np.zeros(f.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)       # 0..8; 8 == smallest normal
    nrm = ~sub
    _, ex = np.frexp(a[nrm])
    e = ex - 1                                                      # floor(log2 a)
    q = np.rint(np.ldexp(a[nrm], -(e - 3))).astype(np.int64)        # 8..16
    carry = q == 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    code[nrm] = ((e + 7) << 3) | (q - 8)
    code = np.minimum(code, 0x7E)                                   # 448 is the largest finite
    code = code | np.where(sign, 0x80, 0)
    code = np.where(np.isnan(f), 0x7F, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------- MXFP4 (OCP MX v1.0)
def decode_e2m1(nib: np.ndarray) -> np.ndarray:
    n = np.asarray(nib).astype(np.int64)
    return np.where(n & 8, -1.0, 1.0) * _E2M1[n & 7]


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """packed [..., C/2] uint8, scales [..., C/32] uint8 -> float64 [..., C]."""
    p = np.asarray(packed)
    lo = decode_e2m1(p & 0xF)
    hi = decode_e2m1(p >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))
    sc = np.asarray(scales).astype(np.int64)
    mult = np.where(sc == 255, np.nan, np.ldexp(1.0, sc - 127))
    mult = np.repeat(mult, 32, axis=-1)
    return vals * mult


def _e2m1_code(v: np.ndarray) -> np.ndarray:
    """Nearest-even E2M1 code (sign in bit 3) of float64 values, saturating to +-6."""
    sign = np.signbit(v)
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.int64)
    sub = a < 1.0
    code[sub] = np.rint(a[sub] / 0.5).astype(np.int64)              # 0, 1 or 2 (2 == 1.0)
    nrm = ~sub
    _, ex = np.frexp(a[nrm])
    e = ex - 1
    q = np.rint(np.ldexp(a[nrm], -(e - 1))).astype(np.int64)        # 2..4
    carry = q == 4
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 2, q)
    c = ((e + 1) << 1) | (q - 2)
    code[nrm] = np.where(e >= 3, 7, c)
    code = np.minimum(code, 7)
    return code | np.where(sign, 8, 0)


def encode_mxfp4(x: np.ndarray):
    """float32 [..., C] (C % 32 == 0) -> (packed [..., C/2] uint8, scales [..., C/32] uint8)."""
    f = np.asarray(x, dtype=np.float32).astype(np.float64)
    C = f.shape[-1]
    assert C % 32 == 0
    g = f.reshape(f.shape[:-1] + (C // 32, 32))
    amax = np.abs(g).max(axis=-1)
    X = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])
    X[nz] = np.clip((ex - 1) - 2, -127, 127)
    v = np.ldexp(g, -X[..., None])
    codes = _e2m1_code(v).reshape(f.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (X + 127).astype(np.uint8)
    return packed, scales


# ----------------------------------------------------------------- stored tensors
class Stored:
    """A tensor kept in its storage format; indexing returns the decoded float64 values.

    ``bits`` is indexed over its leading (row) axes only, so large caches are decoded
    one gathered slice at a time.
    """

    def __init__(self, bits: np.ndarray, dtype: str, scales: np.ndarray | None = None):
        self.bits, self.dtype, self.scales = bits, dtype, scales

    @property
    def shape(self):
        if self.dtype == MXFP4:
            return self.bits.shape[:-1] + (self.bits.shape[-1] * 2,)
        return self.bits.shape

    def __getitem__(self, key):
        return decode(self.bits[key], self.dtype, None if self.scales is None else self.scales[key])


# ----------------------------------------------------------------- FP8 K/V rows
# pogovet.com, 상세 정리 §5: most of each KV entry is stored in FP8 and only the RoPE
# dimensions in BF16.  Reading of what the page leaves open: the RoPE dims are the last
# d_rope dims of a K row (V carries none), the FP8 format is OCP E4M3, and one scale per
# tensor kind maps codes to values (decoded = scale * e4m3(code)).
def decode_fp8_k_rows(rows_u8: np.ndarray, D: int, d_rope: int, k_scale: float) -> np.ndarray:
    """K rows of D - d_rope E4M3 code bytes followed by d_rope little-endian bf16 values
    -> float64 [..., D]: k_scale * code value for the code dims, the bf16 values as they are."""
    r = np.asarray(rows_u8, dtype=np.uint8)
    dn = D - d_rope
    if r.shape[-1] != dn + 2 * d_rope:
        raise ValueError("a K row holds D - d_rope code bytes and d_rope bf16 values")
    codes = r[..., :dn]
    tail = np.ascontiguousarray(r[..., dn:]).view("<u2")
    return np.concatenate([float(k_scale) * decode_e4m3(codes), decode_bf16(tail)], axis=-1)


def decode_fp8_v_rows(rows_u8: np.ndarray, v_scale: float) -> np.ndarray:
    """V rows of D E4M3 code bytes -> float64 [..., D] = v_scale * code value."""
    return float(v_scale) * decode_e4m3(np.asarray(rows_u8, dtype=np.uint8))


def encode_fp8_k_rows(k: np.ndarray, d_rope: int, k_scale: float) -> np.ndarray:
    """float32 K [..., D] -> the byte rows decode_fp8_k_rows reads: e4m3(k / k_scale) for
    the first D - d_rope dims (float32 division, then nearest-even), bf16 of the rest."""
    k = np.asarray(k, dtype=np.float32)
    dn = k.shape[-1] - d_rope
    codes = encode_e4m3(k[..., :dn] / np.float32(k_scale))
    tail = encode_bf16(k[..., dn:]).astype("<u2").view(np.uint8)
    return np.concatenate([codes, tail.reshape(k.shape[:-1] + (2 * d_rope,))], axis=-1)


def encode_fp8_v_rows(v: np.ndarray, v_scale: float) -> np.ndarray:
    """float32 V [..., D] -> E4M3 codes of v / v_scale (float32 division, nearest-even)."""
    return encode_e4m3(np.asarray(v, dtype=np.float32) / np.float32(v_scale))


def decode(bits: np.ndarray, dtype: str, scales: np.ndarray | None = None) -> np.ndarray:
    if dtype == F32:
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return decode_bf16(bits)
    if dtype == FP8_E4M3:
        return decode_e4m3(bits)
    if dtype == MXFP4:
        return decode_mxfp4(bits, scales)
    raise ValueError(dtype)


def rows(t, b, sel) -> np.ndarray:
    """Gather rows ``sel`` of sequence ``b`` of a float64 array or a Stored tensor."""
    return np.asarray(t[b, sel], dtype=np.float64)

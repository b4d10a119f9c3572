"""Number formats and quantisers of the oracle -- TEST INFRASTRUCTURE ONLY.

Formats (definitions, not taken from any implementation):
  * bf16: IEEE binary32 truncated to 8 significant bits; every conversion
    here rounds to nearest, ties to even, directly from the source value.
  * E4M3 ("OCP 8-bit floating point", E4M3FN variant): 1 sign, 4 exponent
    (bias 7), 3 mantissa bits; no infinities; S.1111.111 is NaN; largest
    finite value 448; subnormals m * 2^-9.
  * E2M1 (OCP microscaling FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit;
    magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
Encoders round to nearest, ties to even, and saturate finite values to the
largest magnitude.  The sign bit of a code is set iff the input is < 0 (so a
negative value that rounds to zero gives the negative-zero code).

Quantisation recipes.  The pages fix only the formats: FP8 experts use E4M3
codes with one scalar scale for weights and activations (W8A8), and the
4-bit experts quantise weights and activations alike (W4A4) (bloomery issue
#967, section 2 "Checkpoint facts"; section 6 keeps each release's
activation rules).  The block size (16), the E4M3 block scale and the fp32
tensor scale of the 4-bit format, and the dynamic per-tensor activation
scale, are readings of the layer description, chosen as the plainest ones
consistent with it.  Every step is a named IEEE
float32 operation so that two independent implementations reach identical
codes from identical inputs:

  FP8 per tensor:   s = f32(amax / 448); inv = f32(448 / amax);
                    q = E4M3(f32(v * inv));           value = dec(q) * s
  NVFP4 per tensor: S = f32(amax / 2688)              (2688 = 6 * 448)
                    per 16-block along K: sb = E4M3(f32(amax_b / f32(6 * S)))
                    sb == 0 -> block all zero; else r = f32(1 / f32(dec(sb) * S))
                    q = E2M1(f32(v * r));             value = dec(q) * dec(sb) * S
  amax == 0 gives all-zero codes and a zero scale.

Parity pins (tests/test_codecs.py): exhaustive decode tables against
hand-written tables in tests/golden, every rounding midpoint, saturation,
round trips of every representable value, bf16 against torch's conversion,
hand-derived worked quantiser examples.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
NVFP4_BLOCK = 16


# --------------------------------------------------------------------------- bf16
def bf16_rne(v) -> np.ndarray:
    """Round float64/float32 values to bf16 (nearest, ties to even), returned as float64."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)  # |v| in [2^(e-1), 2^e)
    e = np.maximum(e, -125)  # below 2^-126 the bf16 quantum stays 2^-133
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)


def bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that are exactly bf16."""
    f = np.asarray(v, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- E4M3
def e4m3_decode_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3_decode_table()


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def _round_to_grid(a: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round non-negative float64 `a` to a float grid with `mant_bits` stored
    mantissa bits whose smallest normal is 2^(min_exp-1) (nearest, ties even)."""
    _, e = np.frexp(a)
    e = np.maximum(e, min_exp)
    return np.ldexp(np.rint(np.ldexp(a, mant_bits + 1 - e)), e - mant_bits - 1)


def e4m3_encode(v) -> np.ndarray:
    """E4M3 codes (uint8) of finite values, nearest-even, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    neg = v < 0
    a = np.minimum(np.abs(v), E4M3_MAX)
    r = _round_to_grid(a, 3, -5)  # smallest normal 2^-6
    # map the rounded magnitude back to its code
    sub = r < 2.0 ** -6
    code = np.zeros(r.shape, dtype=np.int64)
    code[sub] = np.rint(r[sub] * 2.0 ** 9).astype(np.int64)
    nr = r[~sub]
    m, e = np.frexp(nr)  # nr = m 2^e, m in [0.5, 1)
    exp_field = (e - 1) + 7
    mant = np.rint((m * 2.0 - 1.0) * 8.0).astype(np.int64)
    code[~sub] = (exp_field << 3) | mant
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- E2M1
def e2m1_decode_table() -> np.ndarray:
    t = np.empty(16, dtype=np.float64)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        t[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return t


_E2M1 = e2m1_decode_table()


def e2m1_decode(codes) -> np.ndarray:
    return _E2M1[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode(v) -> np.ndarray:
    """E2M1 codes (uint8, low nibble) of finite values, nearest-even, saturating at 6."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e2m1_encode: non-finite input")
    neg = v < 0
    a = np.minimum(np.abs(v), E2M1_MAX)
    r = _round_to_grid(a, 1, 1)  # smallest normal 1.0, subnormal step 0.5
    grid = _E2M1[:8]  # 0, 0.5, 1, 1.5, 2, 3, 4, 6: code = position on the grid
    code = np.searchsorted(grid, r).astype(np.int64)
    if not np.array_equal(grid[np.minimum(code, 7)], r):
        raise AssertionError("e2m1_encode: rounded value off the grid")
    code = code | np.where(neg, 0x8, 0)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- recipes
def _amax32(v: np.ndarray) -> np.float32:
    return np.float32(np.max(np.abs(v))) if v.size else np.float32(0.0)


def fp8_quantize(v):
    """Per-tensor E4M3 quantisation of bf16-valued `v` (any shape).

    Returns (codes uint8, scale float32)."""
    v32 = np.asarray(v, dtype=np.float32)
    amax = _amax32(v32)
    if amax == 0:
        return np.zeros(v32.shape, np.uint8), np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    inv = np.float32(np.float32(E4M3_MAX) / amax)
    prod = (v32 * inv).astype(np.float32)
    return e4m3_encode(prod), s


def fp8_dequantize(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.float64(np.float32(scale))


def nvfp4_quantize(v, amax=None):
    """Per-tensor NVFP4 quantisation along the last axis (16-element blocks).

    `amax` overrides the tensor amax (used when one tensor is quantised in
    pieces).  Returns (codes uint8 [..., K] one per element, block scale codes
    uint8 [..., K/16], tensor scale S float32)."""
    v32 = np.asarray(v, dtype=np.float32)
    K = v32.shape[-1]
    if K % NVFP4_BLOCK:
        raise ValueError("nvfp4_quantize: last dim must be a multiple of 16")
    a_t = _amax32(v32) if amax is None else np.float32(amax)
    shape_b = v32.shape[:-1] + (K // NVFP4_BLOCK,)
    if a_t == 0:
        return np.zeros(v32.shape, np.uint8), np.zeros(shape_b, np.uint8), np.float32(0.0)
    S = np.float32(a_t / np.float32(6.0 * E4M3_MAX))
    sixS = np.float32(np.float32(6.0) * S)
    blocks = v32.reshape(shape_b + (NVFP4_BLOCK,))
    amax_b = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    sb_code = e4m3_encode((amax_b / sixS).astype(np.float32))
    sb = e4m3_decode(sb_code).astype(np.float32)  # exact
    den = (sb * S).astype(np.float32)
    live = sb != 0
    r = np.zeros_like(den)
    r[live] = (np.float32(1.0) / den[live]).astype(np.float32)
    prod = (blocks * r[..., None]).astype(np.float32)
    q = e2m1_encode(prod)
    q[~live] = 0
    return q.reshape(v32.shape), sb_code, S


def nvfp4_dequantize(codes, sb_code, S) -> np.ndarray:
    q = e2m1_decode(codes)
    sb = e4m3_decode(sb_code)
    K = q.shape[-1]
    blocks = q.reshape(q.shape[:-1] + (K // NVFP4_BLOCK, NVFP4_BLOCK))
    return (blocks * sb[..., None] * np.float64(np.float32(S))).reshape(q.shape)


def nvfp4_pack(codes) -> np.ndarray:
    """Pack one-per-byte E2M1 codes [..., K] into [..., K/2]: element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def nvfp4_unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out

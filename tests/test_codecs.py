"""Pins for the oracle's number formats and quantiser recipes (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 0), float(v)))
    return rows


# ---------------------------------------------------------------- E2M1
def test_e2m1_table_matches_hand_written():
    t = codecs.e2m1_decode_table()
    rows = _read_table("e2m1_values.txt")
    assert len(rows) == 16
    for c, v in rows:
        assert t[c] == v and np.signbit(t[c]) == np.signbit(v), c


def test_e2m1_midpoints_round_to_even():
    # ties of the E2M1 grid go to the even mantissa
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in ties.items():
        assert codecs.e2m1_decode(codecs.e2m1_encode(np.array([x])))[0] == want, x
        assert codecs.e2m1_decode(codecs.e2m1_encode(np.array([-x])))[0] == -want, x
    # just off the ties, nearest wins
    eps = 1e-6
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for lo, hi in zip(grid[:-1], grid[1:]):
        mid = (lo + hi) / 2
        assert codecs.e2m1_decode(codecs.e2m1_encode(np.array([mid - eps])))[0] == lo
        assert codecs.e2m1_decode(codecs.e2m1_encode(np.array([mid + eps])))[0] == hi


def test_e2m1_saturates_and_round_trips():
    assert list(codecs.e2m1_encode(np.array([6.0, 6.5, 100.0, -7.0, 1e30]))) == [7, 7, 7, 15, 7]
    for c in range(16):
        if c == 8:  # -0 encodes as +0 (sign set only for v < 0)
            continue
        v = codecs.e2m1_decode_table()[c]
        assert codecs.e2m1_encode(np.array([v]))[0] == c
    assert codecs.e2m1_encode(np.array([-0.1]))[0] == 8  # negative rounding to zero keeps the sign


# ---------------------------------------------------------------- E4M3
def test_e4m3_anchors():
    t = codecs.e4m3_decode_table()
    for c, v in _read_table("e4m3_anchors.txt"):
        if np.isnan(v):
            assert np.isnan(t[c]), c
        else:
            assert t[c] == v and np.signbit(t[c]) == np.signbit(v), c


def test_e4m3_table_matches_torch_float8():
    # an independent implementation of the same OCP format
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    t = codecs.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(t))
    assert np.array_equal(ref[~nan], t[~nan])
    assert nan.sum() == 2


def test_e4m3_round_trip_every_code():
    t = codecs.e4m3_decode_table()
    for c in range(256):
        if np.isnan(t[c]) or c == 0x80:
            continue
        assert codecs.e4m3_encode(np.array([t[c]]))[0] == c, hex(c)


def test_e4m3_midpoints_ties_to_even():
    t = codecs.e4m3_decode_table()
    pos = [t[c] for c in range(0x7F)]  # 0 .. 448 ascending
    for c in range(len(pos) - 1):
        lo, hi = pos[c], pos[c + 1]
        mid = (lo + hi) / 2
        got = codecs.e4m3_encode(np.array([mid]))[0]
        want = c if c % 2 == 0 else c + 1  # even code = even mantissa
        assert got == want, (lo, hi)
        assert codecs.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0] == c
        assert codecs.e4m3_encode(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1


def test_e4m3_saturation():
    got = codecs.e4m3_encode(np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, -1e30]))
    assert list(got) == [0x7E] * 6 + [0xFE]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(50),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000).astype(np.float32),
        rng.uniform(-463.0, 463.0, 20000).astype(np.float32),
    ])
    ours = codecs.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of values rounding to zero the same way
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- bf16
def test_bf16_matches_torch_on_float32():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    # force exact ties on part of the sample
    bits[:50000] = (bits[:50000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    ours = codecs.bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)


def test_bf16_rounds_directly_from_float64():
    # 1 + 2^-8 + 2^-40 lies just above the bf16 midpoint; rounding through
    # float32 first would land on the tie and go down to 1.0
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert codecs.bf16_rne(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert codecs.bf16_rne(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert codecs.bf16_rne(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2 * 2.0 ** -7


# ---------------------------------------------------------------- recipes
def test_fp8_recipe_worked_example():
    # amax = 3: s = f32(3/448), inv = f32(448/3) = 149.33333...
    v = np.array([3.0, -1.5, 0.5, 0.0, -3.0], dtype=np.float32)
    q, s = codecs.fp8_quantize(v)
    assert s == np.float32(3.0) / np.float32(448.0)
    # 3*inv ~ 448 -> 0x7E; -1.5*inv ~ -224 (= -1.75*128); 0.5*inv = 74.67 lies
    # between 72 and 80 (step 8 in [64, 128)) and is nearer 72
    assert q[0] == 0x7E and q[4] == 0xFE
    assert codecs.e4m3_decode(q[1]) == -224.0
    assert codecs.e4m3_decode(q[2]) == 72.0
    assert q[3] == 0


def test_fp8_zero_tensor():
    q, s = codecs.fp8_quantize(np.zeros((4, 4), np.float32))
    assert s == 0 and not q.any()


def test_nvfp4_recipe_worked_example():
    # Tensor amax 6 -> S = 6/2688; block 0 has amax 6 -> sb = E4M3(448) = 448,
    # r = 1/(448 S) = 1 -> grid values are kept.  Block 1 has amax 3 ->
    # sb = E4M3(224) = 224, r = 1/(224 S) = 2 -> codes of 2v.
    b0 = np.array([6, -4, 3, 2, 1.5, 1, 0.5, 0, -0.5, -1, -1.5, -2, -3, 4, 6, -6], np.float32)
    b1 = np.array([3, 1.5, 0.75, 0.25, -3, 0, 2, 1, 0.5, -1, 1.25, 2.5, -2.5, 0.125, 1.75, -0.75], np.float32)
    v = np.concatenate([b0, b1])[None, :]
    q, sb, S = codecs.nvfp4_quantize(v)
    assert S == np.float32(6.0) / np.float32(2688.0)
    assert codecs.e4m3_decode(sb[0, 0]) == 448.0
    assert codecs.e4m3_decode(sb[0, 1]) == 224.0
    assert np.array_equal(codecs.e2m1_decode(q[0, :16]), b0.astype(np.float64))
    want1 = [6, 3, 1.5, 0.5, -6, 0, 4, 2, 1, -2, 2, 4, -4, 0, 4, -1.5]  # E2M1(2v), ties to even
    assert np.array_equal(codecs.e2m1_decode(q[0, 16:]), np.array(want1, np.float64))
    deq = codecs.nvfp4_dequantize(q, sb, S)
    s64 = np.float64(S)
    assert np.allclose(deq[0, :16], b0 * 448.0 * s64, rtol=0, atol=0)


def test_nvfp4_exact_round_trip_of_representable_values():
    # Tensor amax 2.625 = 2688 * 2^-10 makes S = 2^-10 exactly; each block holds
    # E2M1 values times an E4M3 scale sb with one element of magnitude 6, so
    # amax_b / (6 S) = sb exactly and the codes come back unchanged.
    rng = np.random.default_rng(3)
    grid = codecs.e2m1_decode_table()[:8]
    n_blocks = 64
    sbv = codecs.e4m3_decode_table()[rng.integers(0x08, 0x7E, n_blocks)]
    sbv[0] = 448.0
    q = grid[rng.integers(0, 8, (n_blocks, 16))] * np.where(rng.random((n_blocks, 16)) < 0.5, -1, 1)
    q[:, 3] = -6.0
    vals64 = q * sbv[:, None] * 2.0 ** -10
    vals = vals64.astype(np.float32)
    assert np.array_equal(vals.astype(np.float64), vals64)  # exactly representable
    codes, sb, S = codecs.nvfp4_quantize(vals.reshape(1, -1))
    assert S == np.float32(2.0 ** -10)
    assert np.array_equal(codecs.e4m3_decode(sb.reshape(-1)), sbv)
    assert np.array_equal(codecs.nvfp4_dequantize(codes, sb, S).reshape(-1), vals64.reshape(-1))


def test_nvfp4_zero_block_and_tensor():
    v = np.zeros((2, 32), np.float32)
    v[0, 16:] = 1.0
    q, sb, S = codecs.nvfp4_quantize(v)
    assert sb[0, 0] == 0 and not q[0, :16].any() and not q[1].any()
    q, sb, S = codecs.nvfp4_quantize(np.zeros((1, 16), np.float32))
    assert S == 0 and not q.any() and not sb.any()


def test_nvfp4_pack_layout():
    c = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    p = codecs.nvfp4_pack(c)
    assert list(p[0]) == [0x21, 0x43, 0x0F]
    assert np.array_equal(codecs.nvfp4_unpack(p), c)


def test_codecs_reject_non_finite():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([np.nan]))
    with pytest.raises(ValueError):
        codecs.e2m1_encode(np.array([np.inf]))

"""Pins of the oracle's MXFP8 rule against references it does not compute itself.

* a hand-computed fixture of blocks (tests/golden/mxfp8_blocks.txt);
* an integer brute force: the nearest finite E4M3 value, ties to the even
  code, found by exhaustive search over the format's code table, for every
  finite bf16 input at several shared exponents;
* PyTorch's float8_e4m3fn conversion (round to nearest even) after clamping
  to +-448, and its decoding of every code;
* the shared exponent recomputed from bf16 exponent bits;
* the MX error bound: |decode(code) * 2^X - v| <= half an E4M3 step of q.
"""

import os

import numpy as np
import pytest
import torch

from oracle import mxfp8

HERE = os.path.dirname(os.path.abspath(__file__))


def expand(tokens):
    out = []
    for t in tokens:
        v, _, n = t.partition("*")
        out += [int(v, 16)] * (int(n) if n else 1)
    return out


def read_blocks():
    blocks, cur = [], None
    with open(os.path.join(HERE, "golden", "mxfp8_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "block":
                cur = {"name": rest}
                blocks.append(cur)
            elif key == "in":
                cur["in"] = expand(rest.split())
            elif key == "scale":
                cur["scale"] = int(rest, 16)
            elif key == "out":
                cur["out"] = expand(rest.split())
    return blocks


@pytest.mark.parametrize("blk", read_blocks(), ids=lambda b: b["name"])
def test_hand_computed_blocks(blk):
    bits = np.array(blk["in"], dtype=np.uint16)[None, :]
    codes, scales = mxfp8.quantize(bits)
    assert scales[0, 0] == blk["scale"]
    np.testing.assert_array_equal(codes[0], np.array(blk["out"], dtype=np.uint8))


def test_short_block_in_a_row():
    """K = 40: the second block holds 8 elements and ignores the first block."""
    bits = np.array([0x3FFF] * 32 + [0x3F80] * 8, dtype=np.uint16)[None, :]
    codes, scales = mxfp8.quantize(bits)
    assert list(scales[0]) == [0x77, 0x77]
    assert list(codes[0, 32:]) == [0x78] * 8


def finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF].astype(np.uint16)


def grid_units():
    """E4M3 finite magnitudes in units of 2^-9, codes 0..0x7E (format definition)."""
    c = np.arange(0x7F)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0)).astype(np.int64)


def brute_codes(bits, X):
    """Nearest finite E4M3 code to v * 2^-X, ties to the even code, by search."""
    b = bits.astype(np.int64)
    E = (b >> 7) & 0xFF
    man = b & 0x7F
    M = np.where(E == 0, man, 128 + man)
    k = np.where(E == 0, -133, E - 134)          # |v| = M * 2^k
    j = k - X + 9                                 # |q| in units of 2^-9 = M * 2^j
    C = grid_units()
    out = np.zeros(b.shape, dtype=np.int64)
    big = (j >= 0) & (j < 40)
    big_val = np.where(big, M << np.clip(j, 0, 39), 0)
    sat = (j >= 40) | (big & (big_val >= C[-1]))
    tiny = j < -30
    rest = ~sat & ~tiny & (M > 0)
    A = np.where(j >= 0, M << np.clip(j, 0, 30), M)[rest]
    r = np.clip(-j, 0, 30)[rest]
    D = np.abs(A[:, None] - (C[None, :] << r[:, None]))
    mn = D.min(1)
    cand = D == mn[:, None]
    even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    pick = np.where(even.any(1), even.argmax(1), cand.argmax(1))
    out[rest] = pick
    out[sat & (M > 0)] = 0x7E
    sign = np.where(b & 0x8000, 0x80, 0)
    return (out | sign).astype(np.uint8)


@pytest.mark.parametrize("X", [-127, -20, -13, -8, 0, 60, 119] +
                         list(np.random.default_rng(11).integers(-127, 120, 6)))
def test_encode_exhaustive_vs_brute_force(X):
    bits = finite_bf16()
    v = mxfp8.bf16_bits_to_f64(bits)
    got = mxfp8.e4m3_encode(np.ldexp(v, -int(X)))
    want = brute_codes(bits, int(X))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(bits[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("X", [-127, -13, -8, 0, 30, 119])
def test_encode_vs_torch_float8(X):
    bits = finite_bf16()
    v = mxfp8.bf16_bits_to_f64(bits)
    q = np.ldexp(v, -X)
    got = mxfp8.e4m3_encode(q)
    qt = torch.from_numpy(np.clip(q, -448.0, 448.0).astype(np.float32))
    want = qt.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(bits[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mxfp8.e4m3_decode(codes)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_grid_units_match_decode():
    np.testing.assert_array_equal(grid_units(), mxfp8.e4m3_decode(np.arange(0x7F)) * 512)


def bits_exponent(amax_bits):
    """floor(log2) of a positive bf16 magnitude from its exponent / mantissa bits."""
    E = (amax_bits >> 7) & 0xFF
    m = amax_bits & 0x7F
    sub = np.floor(np.log2(np.maximum(m, 1))).astype(np.int64) - 133
    return np.where(E == 0, sub, E.astype(np.int64) - 127)


def random_blocks(rng, n):
    """Blocks of bf16 bits: N(0, s) with s spread over many binades, some zeros,
    negative zeros and subnormals."""
    scale = np.exp2(rng.integers(-140, 120, size=(n, 1))).astype(np.float64)
    x = rng.standard_normal((n, 32)) * scale
    x = np.clip(x, -3e38, 3e38).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    b[rng.random((n, 32)) < 0.05] = 0
    b[rng.random((n, 32)) < 0.05] = 0x8000
    b[rng.random((n, 32)) < 0.05] = rng.integers(1, 0x80, size=1)[0]
    return b


def test_scale_rule_from_exponent_bits():
    rng = np.random.default_rng(5)
    blocks = random_blocks(rng, 4000)
    _, scales = mxfp8.quantize(blocks)
    amax_bits = (blocks & 0x7FFF).max(axis=1).astype(np.int64)
    want = np.where(amax_bits == 0, -127,
                    np.clip(bits_exponent(amax_bits) - 8, -127, 127)) + 127
    np.testing.assert_array_equal(scales[:, 0], want.astype(np.uint8))


def test_blocks_vs_brute_force_and_error_bound():
    rng = np.random.default_rng(6)
    blocks = random_blocks(rng, 3000)
    codes, scales = mxfp8.quantize(blocks)
    X = scales[:, 0].astype(np.int64) - 127
    for i in range(0, 3000, 7):
        np.testing.assert_array_equal(codes[i], brute_codes(blocks[i], int(X[i])))
    v = mxfp8.bf16_bits_to_f64(blocks)
    q = np.ldexp(v, -X[:, None])
    dec = mxfp8.e4m3_decode(codes)
    inside = np.abs(q) < 448
    k = np.maximum(np.floor(np.log2(np.where(np.abs(q) > 0, np.abs(q), 1))), -6)
    half_step = np.exp2(k - 4)
    assert (np.abs(dec - q)[inside] <= half_step[inside]).all()
    assert (np.abs(q) < 512).all()


def test_nan_block_convention():
    """Convention only (no page fixes it): NaN/Inf block -> scale 0xFF, elements 0x7F."""
    bits = np.array([[0x7FC0] + [0x3F80] * 31, [0xFF80] + [0] * 31], dtype=np.uint16)
    codes, scales = mxfp8.quantize(bits)
    assert list(scales[:, 0]) == [0xFF, 0xFF]
    assert (codes == 0x7F).all()


def test_normal_002_clip_fraction():
    """Under N(0, 0.02) roughly a fifth of 32-element blocks clip their largest
    element (amax * 2^-X lands in [448, 512)): a property of the floor scale."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((20000, 32)) * 0.02).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    codes, _ = mxfp8.quantize(b)
    frac = ((codes & 0x7F) == 0x7E).any(axis=1).mean()
    assert 0.1 < frac < 0.3

"""BF16 -> MXFP8 quantisation rule (oracle; test infrastructure only).

"NCCL Reshard Refit (Experimental)", section "Enabling It": with BF16 training
and MXFP8 generation, the generation side quantises each received BF16 shard
before installing it.  The pages do not give the format's arithmetic, so the
oracle follows the OCP Microscaling Formats (MX) v1.0 specification for
MXFP8 E4M3 (shared-scale conversion, its section 6.3), with these choices:

  * block: 32 consecutive elements along the destination shard's last
    dimension, counted from local column 0; a short last block uses only its
    valid elements;
  * shared scale X = floor(log2(amax)) - 8 (8 is E4M3's largest normal
    exponent), clamped to [-127, 127]; an all-zero block takes X = -127;
    the scale byte is the E8M0 encoding X + 127;
  * element = E4M3 encoding of v * 2^-X, round to nearest with ties to even,
    saturating to +-448 (code 0x7E / 0xFE) instead of overflowing;
  * the sign of zero is kept (negative values that round to zero give 0x80);
  * a block holding a NaN or an infinity gets scale 0xFF and every element
    0x7F (a convention: no page fixes it).

All arithmetic below is exact: bf16 values, powers of two and the E4M3 grid
are all representable in float64 over the ranges reached here.
"""

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E
SCALE_NAN = 0xFF
ELEM_NAN = 0x7F


def bf16_bits_to_f64(bits):
    """Exact float64 values of bfloat16 bit patterns (uint16 array)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # signalling NaN patterns widen to quiet NaNs
        return b.view(np.float32).astype(np.float64)


def floor_log2(x):
    """floor(log2(x)) for positive finite float64 values, exactly (via frexp)."""
    _, e = np.frexp(x)
    return e.astype(np.int64) - 1


def shared_exponent(amax):
    """X = clamp(floor(log2(amax)) - 8, -127, 127); amax == 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    out[nz] = np.clip(floor_log2(amax[nz]) - 8, -127, 127)
    return out


def e4m3_encode(q):
    """Saturating round-to-nearest-even E4M3 code of each (exact) float64 q.

    E4M3 (bias 7): subnormals are m * 2^-9 (m = 0..7); normals are
    (1 + m/8) * 2^(e-7) for e = 1..15, with code 0x7F reserved for NaN, so
    the largest finite magnitude is 448 (code 0x7E).  Within binade
    [2^k, 2^(k+1)) the grid step is 2^(k-3); below 2^-6 it is 2^-9.
    """
    q = np.asarray(q, dtype=np.float64)
    t = np.abs(q)
    sign = np.where(np.signbit(q), 0x80, 0x00).astype(np.int64)
    code = np.zeros(q.shape, dtype=np.int64)
    sat = t >= E4M3_MAX
    fin = (~sat) & (t > 0)
    k = np.maximum(floor_log2(np.where(fin, t, 1.0)), -6)
    step_exp = k - 3
    n = np.rint(np.ldexp(np.where(fin, t, 0.0), -step_exp))   # exact scaling, RNE
    c = (k + 6) * 8 + n.astype(np.int64)          # a carry of n to 16 moves to the next binade
    code = np.where(fin, np.minimum(c, E4M3_MAX_CODE), code)
    code = np.where(sat, E4M3_MAX_CODE, code)
    return (code | sign).astype(np.uint8)


def e4m3_decode(codes):
    """float64 value of E4M3 codes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def quantize(bits):
    """Quantise bf16 bit patterns of shape [..., K] along the last dimension.

    Returns (codes uint8 [..., K], scales uint8 [..., ceil(K/32)]).
    """
    bits = np.asarray(bits, dtype=np.uint16)
    shape = bits.shape
    K = shape[-1]
    nb = -(-K // BLOCK)
    v = bf16_bits_to_f64(bits)
    codes = np.zeros(shape, dtype=np.uint8)
    scales = np.zeros(shape[:-1] + (nb,), dtype=np.uint8)
    for b in range(nb):
        lo, hi = b * BLOCK, min((b + 1) * BLOCK, K)
        vb = v[..., lo:hi]
        bad = ~np.isfinite(vb).all(axis=-1)
        amax = np.max(np.abs(np.where(np.isfinite(vb), vb, 0.0)), axis=-1)
        X = shared_exponent(amax)
        q = np.ldexp(vb, -X[..., None])
        cb = e4m3_encode(q)
        cb[bad] = ELEM_NAN
        codes[..., lo:hi] = cb
        sb = (X + 127).astype(np.uint8)
        sb[bad] = SCALE_NAN
        scales[..., b] = sb
    return codes, scales

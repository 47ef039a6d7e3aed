"""Number formats and block quantizers, in plain NumPy fp64.

Test infrastructure only (see the package docstring).

Formats (TEARDOWN "What is 4-bit"; LAYER "Model profile" rows "Expert
formats" and "D/U formats"):

* NVFP4 expert weights: FP4 (E2M1) values, one E4M3 scale per 16 values,
  plus a 16-byte tail per record. Our reading of the tail: the fp32 per-matrix
  tensor scale of gate, up and down, then 4 zero bytes.
* Q8 / Q4 D/U: 8-bit or 4-bit integer codes with one fp16 scale per 32
  values. The byte totals the teardown prints (47.79 GiB, 32.96 GiB, 1.42 GB)
  fix 34 B and 18 B per 32 weights.
* bf16 router and shared-expert weights (TEARDOWN "The base, byte for byte").

Readings where the pages are silent: blocks run along the reduction (input)
dimension of each weight row; element 2i sits in the low nibble of byte i;
every rounding is round-to-nearest-even and saturating.
"""

import numpy as np

# ---------------------------------------------------------------------------
# Generic rounding to a binary floating-point grid.


def round_pos(v, mant_bits, emin):
    """Round non-negative fp64 ``v`` to the nearest value with ``mant_bits``
    fraction bits and exponent >= ``emin`` (subnormal spacing below 2**emin),
    ties to even. No saturation here; callers clamp.

    Exact in fp64 for the formats used: the scaled value is an integer of at
    most 12 bits after ``rint``, and ``ldexp`` is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)                    # v = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, emin)           # exponent of the leading bit
    q = np.rint(np.ldexp(v, mant_bits - e))  # numpy rint is half-to-even
    out = np.ldexp(q, e - mant_bits)
    return np.where(v == 0, 0.0, out)


# ---------------------------------------------------------------------------
# E2M1 (FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit.


def e2m1_decode(codes):
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e2m1_encode(v):
    """RNE to E2M1, saturating at +-6. A value whose magnitude rounds to zero
    encodes as +0 (code 0), whatever its sign."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(round_pos(np.abs(v), 1, 0), 6.0)
    # magnitude -> 3-bit code: e = 0 holds 0 and 0.5; else 2**(e-1)*(1+m/2)
    _, ex = np.frexp(np.where(mag == 0, 1.0, mag))
    e = np.where(mag < 1.0, 0, ex)                 # mag in [2**(e-1), 2**e)
    m = np.where(e == 0, np.rint(mag * 2.0),
                 np.rint((np.ldexp(mag, -(e - 1).astype(np.int64)) - 1.0) * 2.0))
    code = (e.astype(np.int64) << 1) | m.astype(np.int64)
    neg = (v < 0) & (mag != 0)
    return (code | (neg.astype(np.int64) << 3)).astype(np.uint8)


# ---------------------------------------------------------------------------
# E4M3 (OCP E4M3FN): bias 7, no infinities, 0x7F / 0xFF are NaN, max 448.


def e4m3_decode(b):
    b = np.asarray(b).astype(np.int64) & 0xFF
    s = b >> 7
    e = (b >> 3) & 0xF
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(v):
    """RNE of a non-negative value to E4M3, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0):
        raise ValueError("e4m3_encode takes non-negative values (block scales)")
    r = np.minimum(round_pos(v, 3, -6), 448.0)
    _, ex = np.frexp(np.where(r == 0, 1.0, r))
    E = ex - 1                                       # r in [2**E, 2**(E+1))
    sub = r < 2.0 ** -6
    e_field = np.where(sub, 0, E + 7)
    m_field = np.where(sub, np.rint(np.ldexp(r, 9)),
                       np.rint((np.ldexp(r, -E.astype(np.int64)) - 1.0) * 8.0))
    return ((e_field.astype(np.int64) << 3) | m_field.astype(np.int64)).astype(np.uint8)


# ---------------------------------------------------------------------------
# fp16 and bf16 bit patterns.


def f64_to_f16_bits(v):
    """RNE of fp64 to IEEE binary16 (finite inputs below 65504 only)."""
    v = np.asarray(v, dtype=np.float64)
    mag = round_pos(np.abs(v), 10, -14)
    if np.any(mag > 65504.0):
        raise OverflowError("value outside the fp16 range")
    _, ex = np.frexp(np.where(mag == 0, 1.0, mag))
    E = ex - 1
    sub = mag < 2.0 ** -14
    e_field = np.where(sub, 0, E + 15)
    m_field = np.where(sub, np.rint(np.ldexp(mag, 24)),
                       np.rint((np.ldexp(mag, -E.astype(np.int64)) - 1.0) * 1024.0))
    bits = (e_field.astype(np.int64) << 10) | m_field.astype(np.int64)
    bits = bits | (((v < 0) & (mag != 0)).astype(np.int64) << 15)
    return bits.astype(np.uint16)


def f16_bits_to_f64(bits):
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = b >> 15
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    mag = np.where(e == 0, np.ldexp(m / 1024.0, -14), np.ldexp(1.0 + m / 1024.0, e - 15))
    return np.where(s == 1, -mag, mag)


def f32_to_bf16_bits(x):
    """RNE of fp32 values to bfloat16 bit patterns (finite inputs)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    mag = round_pos(np.abs(x), 7, -126)
    _, ex = np.frexp(np.where(mag == 0, 1.0, mag))
    E = ex - 1
    sub = mag < 2.0 ** -126
    e_field = np.where(sub, 0, E + 127)
    m_field = np.where(sub, np.rint(np.ldexp(mag, 133)),
                       np.rint((np.ldexp(mag, -E.astype(np.int64)) - 1.0) * 128.0))
    bits = (e_field.astype(np.int64) << 7) | m_field.astype(np.int64)
    bits = bits | (((x < 0) & (mag != 0)).astype(np.int64) << 15)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# NVFP4: E2M1 codes, E4M3 scale per 16 along the row, fp32 tensor scale.

E2M1_MAX = 6.0
E4M3_MAX = 448.0


def quantize_nvfp4(w):
    """Quantize an fp32 matrix [rows, K] (K % 16 == 0).

    Returns (codes uint8 [rows, K] holding 4-bit codes, scales uint8
    [rows, K/16] E4M3 bytes, ts float32). Reading of the recipe:
      ts  = fp32(amax(W) / (6*448))     (1.0 for an all-zero matrix)
      s_b = RNE_E4M3(amax_b / (6*ts))   saturating at 448
      q   = RNE_E2M1(W / (s_b*ts))      saturating at +-6; s_b = 0 -> q = +0
    so that W ~ e2m1(q) * e4m3(s_b) * ts.
    """
    w = np.asarray(w, dtype=np.float32)
    rows, k = w.shape
    assert k % 16 == 0
    wd = w.astype(np.float64)
    amax = float(np.max(np.abs(wd))) if wd.size else 0.0
    ts = np.float32(amax / (E2M1_MAX * E4M3_MAX)) if amax > 0 else np.float32(1.0)
    blk = wd.reshape(rows, k // 16, 16)
    amax_b = np.max(np.abs(blk), axis=2)
    s_bytes = e4m3_encode(amax_b / (E2M1_MAX * float(ts)))
    s_val = e4m3_decode(s_bytes)
    denom = s_val[:, :, None] * float(ts)
    ratio = np.divide(blk, denom, out=np.zeros_like(blk), where=denom > 0)
    codes = e2m1_encode(ratio).reshape(rows, k)
    codes[np.repeat(s_val == 0, 16, axis=1)] = 0
    return codes, s_bytes, ts


def dequantize_nvfp4(codes, scales, ts):
    rows, k = codes.shape
    v = e2m1_decode(codes).reshape(rows, k // 16, 16)
    v = v * e4m3_decode(scales)[:, :, None] * float(np.float32(ts))
    return v.reshape(rows, k)


def pack_nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def expert_record_bytes(ell, f):
    """Bytes of one NVFP4 expert record: three matrices of ell*f weights at
    4 bits, one E4M3 byte per 16 weights, and a 16-byte tail."""
    n = ell * f
    return 3 * (n // 2) + 3 * (n // 16) + 16


def pack_expert_record(gate, up, down):
    """gate, up: fp32 [F, ell]; down: fp32 [ell, F]. Returns (bytes, parts).

    Section order (our reading; the pages fix only the total): gate codes,
    up codes, down codes (each [rows, K/2] nibble pairs), gate scales, up
    scales, down scales (each [rows, K/16] E4M3), tail (fp32 ts_gate, ts_up,
    ts_down, uint32 0).
    """
    qs = [quantize_nvfp4(m) for m in (gate, up, down)]
    parts = [pack_nibbles(q[0]).ravel() for q in qs]
    parts += [q[1].ravel() for q in qs]
    tail = np.array([q[2] for q in qs] + [np.float32(0)], dtype=np.float32).view(np.uint8)
    tail[12:] = 0
    rec = np.concatenate(parts + [tail]).astype(np.uint8)
    assert rec.size == expert_record_bytes(gate.shape[1], gate.shape[0])
    return rec


def unpack_expert_record(rec, ell, f):
    """Decode a record to fp64 (gate [F, ell], up [F, ell], down [ell, F])."""
    rec = np.asarray(rec, dtype=np.uint8)
    n = ell * f
    if rec.size != expert_record_bytes(ell, f):
        raise ValueError("wrong expert record size")
    off = 0
    codes = []
    for _ in range(3):
        codes.append(unpack_nibbles(rec[off:off + n // 2]))
        off += n // 2
    scales = []
    for _ in range(3):
        scales.append(rec[off:off + n // 16])
        off += n // 16
    ts = rec[off:off + 12].view(np.float32)
    shapes = [(f, ell), (f, ell), (ell, f)]
    mats = []
    for c, s, t, (r, k) in zip(codes, scales, ts, shapes):
        mats.append(dequantize_nvfp4(c.reshape(r, k), s.reshape(r, k // 16), t))
    return mats[0], mats[1], mats[2]


# ---------------------------------------------------------------------------
# Q8 / Q4 blocks of 32 along the row, fp16 scale.


def quantize_blocks(w, bits):
    """Q8: d = fp16(amax_b/127), q = clamp(RNE(x/d), -127, 127), int8.
    Q4: d = fp16(amax_b/7),   q = clamp(RNE(x/d), -8, 7), stored as q+8.
    A block whose d rounds to 0 stores q = 0.
    Returns (codes uint8 [rows, K] (Q8: int8 bit patterns; Q4: nibbles q+8),
    scale bits uint16 [rows, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    rows, k = w.shape
    assert k % 32 == 0 and bits in (8, 4)
    qmax, qmin = (127, -127) if bits == 8 else (7, -8)
    blk = w.astype(np.float64).reshape(rows, k // 32, 32)
    amax_b = np.max(np.abs(blk), axis=2)
    d_bits = f64_to_f16_bits(amax_b / qmax)
    d = f16_bits_to_f64(d_bits)
    ratio = np.divide(blk, d[:, :, None], out=np.zeros_like(blk), where=d[:, :, None] > 0)
    q = np.clip(np.rint(ratio), qmin, qmax).astype(np.int64).reshape(rows, k)
    codes = (q & 0xFF).astype(np.uint8) if bits == 8 else (q + 8).astype(np.uint8)
    return codes, d_bits


def dequantize_blocks(codes, d_bits, bits):
    rows, k = codes.shape
    if bits == 8:
        q = codes.view(np.int8).astype(np.float64)
    else:
        q = codes.astype(np.float64) - 8.0
    d = f16_bits_to_f64(d_bits)
    return (q.reshape(rows, k // 32, 32) * d[:, :, None]).reshape(rows, k)


def du_group_bytes(rows, k, bits):
    """Bytes of one D_g or U_g matrix: codes then fp16 scales."""
    return rows * k * bits // 8 + rows * (k // 32) * 2


def pack_du(w, bits):
    codes, d_bits = quantize_blocks(w, bits)
    c = codes if bits == 8 else pack_nibbles(codes)
    return np.concatenate([c.ravel(), d_bits.ravel().view(np.uint8)]).astype(np.uint8)


def unpack_du(blob, rows, k, bits):
    blob = np.asarray(blob, dtype=np.uint8)
    nc = rows * k * bits // 8
    if blob.size != du_group_bytes(rows, k, bits):
        raise ValueError("wrong D/U group size")
    c = blob[:nc].reshape(rows, k * bits // 8)
    codes = c if bits == 8 else unpack_nibbles(c)
    d_bits = blob[nc:].view(np.uint16).reshape(rows, k // 32)
    return dequantize_blocks(codes.reshape(rows, k), d_bits, bits)

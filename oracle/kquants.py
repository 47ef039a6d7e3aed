"""Q3_K and IQ4_NL expert blocks (the Q3_K builds), plain NumPy.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (see the package docstring).

The pages name the formats of the Q3_K builds and fix their sizes, not their
codes: "Edge0-145B: a Qwen MoE with its experts squeezed, and a 51B table
left on the SSD", section "What is 4-bit" (Q3_K for gate and up, IQ4_NL for
down; 985,600 + 645,120 bytes, a 1,630,720-byte record at latent 1792, 3.79
bits a weight) and the "Edge0 145B and Edge0 120B" model page (1,164,800
bytes a record at latent 1280). The block layouts are GGML's published
Q3_K and IQ4_NL blocks, restated here from their definition:

Q3_K, a super-block of 256 weights along the row, 110 bytes:
  hmask[32]   bit 4h + j of byte 16b + l: the high bit of weight 128h + 32j + 16b + l
  qs[64]      bits 2j, 2j + 1 of byte 32h + 16b + l: its two low bits
  scales[12]  sixteen 6-bit sub-block scales; scale i has its low nibble in
              byte i % 8 (the high nibble of that byte for i >= 8) and its top
              two bits at bits 2 (i // 4), 2 (i // 4) + 1 of byte 8 + i % 4
  d           fp16
  weight 128h + 32j + 16b + l = d * (scale[8h + 2j + b] - 32) * (low2 - (high ? 0 : 4))
  (h in 0..1, j in 0..3, b in 0..1, l in 0..15)

IQ4_NL, a block of 32 weights, 18 bytes: d fp16, then qs[16]; weight l < 16
is d * TABLE[qs[l] & 15], weight 16 + l is d * TABLE[qs[l] >> 4], with the
format's fixed non-uniform table TABLE below.

Record (a reading; only its size is on the pages): gate blocks (row-major,
[F][ell / 256]), up blocks, down blocks ([ell][F / 32]); nothing else (the
"column scales" the model page mentions do not fit in the record's bytes
and are taken as 1).

The quantizers are this module's own (the pages give none):
  Q3_K:   per sub-block of 16, s_b = max(largest value / 3, largest
          magnitude of a negative value / 4) (codes run from -4 to 3);
          d = fp16(max_b s_b / 31);
          scale_b = clamp(RNE(s_b / d), 0, 31) + 32; q = clamp(RNE(x / dl), -4, 3)
          with dl = d (scale_b - 32) (q = 0 where dl = 0)
  IQ4_NL: d = fp16(max(largest value / 113, largest magnitude of a negative
          value / 127)) (the table's ends); each weight to the nearest
          d * TABLE entry (the lower index on a tie)
"""

import numpy as np

from .formats import f16_bits_to_f64, f64_to_f16_bits

IQ4NL_TABLE = np.array([-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113],
                       dtype=np.int64)
Q3K_BYTES = 110
IQ4NL_BYTES = 18


# ---------------------------------------------------------------------------
# Q3_K


def _q3k_index():
    """(h, j, b, l) of each of the 256 weights of a super-block, in order."""
    w = np.arange(256)
    return w // 128, (w % 128) // 32, (w % 32) // 16, w % 16


def q3k_pack_scales(sc):
    """sixteen 6-bit scales [..., 16] -> 12 bytes [..., 12]."""
    sc = np.asarray(sc, dtype=np.int64)
    out = np.zeros(sc.shape[:-1] + (12,), dtype=np.int64)
    for i in range(16):
        lo, hi = sc[..., i] & 15, sc[..., i] >> 4
        out[..., i % 8] |= lo << (4 if i >= 8 else 0)
        out[..., 8 + i % 4] |= hi << (2 * (i // 4))
    return out.astype(np.uint8)


def q3k_unpack_scales(b):
    b = np.asarray(b, dtype=np.int64)
    out = np.zeros(b.shape[:-1] + (16,), dtype=np.int64)
    for i in range(16):
        lo = (b[..., i % 8] >> (4 if i >= 8 else 0)) & 15
        hi = (b[..., 8 + i % 4] >> (2 * (i // 4))) & 3
        out[..., i] = lo | (hi << 4)
    return out


def q3k_quantize(w):
    """fp32 [rows, K] (K % 256 == 0) -> uint8 [rows, K / 256, 110]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    rows, k = w.shape
    assert k % 256 == 0
    sb = w.reshape(rows, k // 256, 16, 16)                  # [.., sub-block, 16]
    s = np.maximum(np.max(sb, axis=3) / 3.0, np.max(-sb, axis=3) / 4.0)
    s = np.maximum(s, 0.0)
    d_bits = f64_to_f16_bits(np.max(s, axis=2) / 31.0)
    d = f16_bits_to_f64(d_bits)
    code = np.clip(np.rint(np.divide(s, d[..., None], out=np.zeros_like(s), where=d[..., None] > 0)),
                   0, 31).astype(np.int64) + 32
    dl = d[..., None] * (code - 32)
    q = np.clip(np.rint(np.divide(sb, dl[..., None], out=np.zeros_like(sb), where=dl[..., None] > 0)),
                -4, 3).astype(np.int64)
    u = (q + 4).reshape(rows, k // 256, 256)               # 3-bit codes, weight order
    h, j, b, l = _q3k_index()
    qs = np.zeros((rows, k // 256, 64), dtype=np.int64)
    hm = np.zeros((rows, k // 256, 32), dtype=np.int64)
    for wi in range(256):
        qs[..., 32 * h[wi] + 16 * b[wi] + l[wi]] |= (u[..., wi] & 3) << (2 * j[wi])
        hm[..., 16 * b[wi] + l[wi]] |= (u[..., wi] >> 2) << (4 * h[wi] + j[wi])
    out = np.zeros((rows, k // 256, Q3K_BYTES), dtype=np.uint8)
    out[..., 0:32] = hm
    out[..., 32:96] = qs
    out[..., 96:108] = q3k_pack_scales(code)
    out[..., 108:110] = d_bits.astype(np.uint16)[..., None].view(np.uint8).reshape(rows, k // 256, 2)
    return out


def q3k_dequantize(blocks):
    """uint8 [rows, nb, 110] -> fp64 [rows, nb * 256]."""
    blk = np.asarray(blocks, dtype=np.uint8)
    rows, nb, _ = blk.shape
    hm = blk[..., 0:32].astype(np.int64)
    qs = blk[..., 32:96].astype(np.int64)
    sc = q3k_unpack_scales(blk[..., 96:108])
    d = f16_bits_to_f64(np.ascontiguousarray(blk[..., 108:110]).view(np.uint16)[..., 0])
    h, j, b, l = _q3k_index()
    out = np.zeros((rows, nb, 256))
    for wi in range(256):
        low = (qs[..., 32 * h[wi] + 16 * b[wi] + l[wi]] >> (2 * j[wi])) & 3
        high = (hm[..., 16 * b[wi] + l[wi]] >> (4 * h[wi] + j[wi])) & 1
        q = low - np.where(high == 1, 0, 4)
        out[..., wi] = d * (sc[..., 8 * h[wi] + 2 * j[wi] + b[wi]] - 32) * q
    return out.reshape(rows, nb * 256)


# ---------------------------------------------------------------------------
# IQ4_NL


def iq4nl_quantize(w):
    """fp32 [rows, K] (K % 32 == 0) -> uint8 [rows, K / 32, 18]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    rows, k = w.shape
    assert k % 32 == 0
    blk = w.reshape(rows, k // 32, 32)
    d_bits = f64_to_f16_bits(np.maximum(np.maximum(np.max(blk, axis=2) / 113.0,
                                                   np.max(-blk, axis=2) / 127.0), 0.0))
    d = f16_bits_to_f64(d_bits)
    vals = d[..., None, None] * IQ4NL_TABLE[None, None, None, :]   # [rows, nb, 1, 16]
    idx = np.argmin(np.abs(blk[..., None] - vals), axis=3)         # first minimum: lower index
    out = np.zeros((rows, k // 32, IQ4NL_BYTES), dtype=np.uint8)
    out[..., 0:2] = d_bits.astype(np.uint16)[..., None].view(np.uint8).reshape(rows, k // 32, 2)
    out[..., 2:18] = (idx[..., :16] | (idx[..., 16:] << 4)).astype(np.uint8)
    return out


def iq4nl_dequantize(blocks):
    blk = np.asarray(blocks, dtype=np.uint8)
    rows, nb, _ = blk.shape
    d = f16_bits_to_f64(np.ascontiguousarray(blk[..., 0:2]).view(np.uint16)[..., 0])
    qs = blk[..., 2:18].astype(np.int64)
    idx = np.concatenate([qs & 15, qs >> 4], axis=2)
    return (d[..., None] * IQ4NL_TABLE[idx]).reshape(rows, nb * 32)


# ---------------------------------------------------------------------------
# Expert record


def q3k_record_bytes(ell, f):
    return 2 * f * (ell // 256) * Q3K_BYTES + ell * (f // 32) * IQ4NL_BYTES


def pack_q3k_record(gate, up, down):
    """gate, up: fp32 [F, ell]; down: fp32 [ell, F] -> the record's bytes."""
    f, ell = gate.shape
    rec = np.concatenate([q3k_quantize(gate).ravel(), q3k_quantize(up).ravel(),
                          iq4nl_quantize(down).ravel()]).astype(np.uint8)
    assert rec.size == q3k_record_bytes(ell, f)
    return rec


def unpack_q3k_record(rec, ell, f):
    """fp64 (gate [F, ell], up [F, ell], down [ell, F])."""
    rec = np.asarray(rec, dtype=np.uint8)
    if rec.size != q3k_record_bytes(ell, f):
        raise ValueError("wrong Q3_K record size")
    n1 = f * (ell // 256) * Q3K_BYTES
    g = q3k_dequantize(rec[:n1].reshape(f, ell // 256, Q3K_BYTES))
    u = q3k_dequantize(rec[n1:2 * n1].reshape(f, ell // 256, Q3K_BYTES))
    dn = iq4nl_dequantize(rec[2 * n1:].reshape(ell, f // 32, IQ4NL_BYTES))
    return g, u, dn

"""Pins of the Q3_K / IQ4_NL oracle ("Edge0-145B: a Qwen MoE with its experts
squeezed, and a 51B table left on the SSD", section "What is 4-bit"; "Edge0
145B and Edge0 120B", architecture tables): the record sizes the pages
print, and the block layouts checked by decoding blocks built bit by bit in
the order the format stores them (an element counter that walks halves,
shift groups, sub-blocks and lanes), independently of the oracle's
closed-form indices."""

import numpy as np
import pytest

from oracle import kquants as kq
from oracle import layer as ol

F16_ONE = 0x3C00


def test_record_sizes_match_the_pages():
    # 985,600 bytes of Q3_K gate and up plus 645,120 of IQ4_NL down
    assert 2 * 640 * (1792 // 256) * kq.Q3K_BYTES == 985600
    assert 1792 * (640 // 32) * kq.IQ4NL_BYTES == 645120
    assert kq.q3k_record_bytes(1792, 640) == 1630720
    assert kq.q3k_record_bytes(1280, 640) == 1164800
    assert round(1630720 * 8 / (3 * 1792 * 640), 2) == 3.79
    assert ol.LayerDims(2560, 1792, 512, 10, 8, 640, 640, 8, expert_format=1).record_bytes == 1630720


def _walk():
    """(sub-block, qs byte, shift, hmask byte, hmask bit) of the 256 weights in
    storage order: two halves of 128, four shift groups of 32 per half, two
    runs of 16 per shift group; the qs pointer advances by 32 per half, the
    hmask bit by one per shift group."""
    out, sb, m = [], 0, 0
    for half in range(2):
        for shift in range(4):
            for run in range(2):
                for l in range(16):
                    out.append((sb, 32 * half + 16 * run + l, 2 * shift, 16 * run + l, m))
                sb += 1
            m += 1
    return out


def _block(d_bits, codes6, u3):
    """A Q3_K block from 16 scale codes and 256 three-bit codes (storage order)."""
    blk = np.zeros(110, dtype=np.uint8)
    for w, (sb, qb, sh, hb, bit) in enumerate(_walk()):
        blk[32 + qb] |= (u3[w] & 3) << sh
        blk[hb] |= (u3[w] >> 2) << bit
    blk[96:108] = kq.q3k_pack_scales(np.asarray(codes6))
    blk[108:110] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    return blk


def test_q3k_layout_by_construction():
    rng = np.random.default_rng(0)
    codes6 = rng.integers(0, 64, 16)
    u3 = rng.integers(0, 8, 256)
    blk = _block(F16_ONE, codes6, u3)
    got = kq.q3k_dequantize(blk[None, None])[0]
    want = [(codes6[sb] - 32) * (u3[w] - 4) for w, (sb, *_r) in enumerate(_walk())]
    np.testing.assert_array_equal(got, want)


def test_q3k_scale_bytes_round_trip_every_value():
    rng = np.random.default_rng(1)
    for i in range(16):
        for v in range(64):
            sc = rng.integers(0, 64, 16)
            sc[i] = v
            assert np.array_equal(kq.q3k_unpack_scales(kq.q3k_pack_scales(sc)), sc)


def test_q3k_high_bit_and_offset():
    """All low bits 3 with every high bit set is +3 everywhere; with none set,
    -1 (the code minus 4)."""
    one = np.full(16, 33)
    blk = _block(F16_ONE, one, np.full(256, 7))
    assert (kq.q3k_dequantize(blk[None, None]) == 3).all()
    blk = _block(F16_ONE, one, np.full(256, 3))
    assert (kq.q3k_dequantize(blk[None, None]) == -1).all()


def test_iq4nl_table_and_layout():
    t = kq.IQ4NL_TABLE
    assert t.size == 16 and (np.diff(t) > 0).all() and t[0] == -127 and t[-1] == 113
    blk = np.zeros(18, dtype=np.uint8)
    blk[0:2] = np.array([0x4000], dtype=np.uint16).view(np.uint8)   # d = 2
    blk[2:] = np.arange(16) | ((15 - np.arange(16)) << 4)
    got = kq.iq4nl_dequantize(blk[None, None])[0]
    np.testing.assert_array_equal(got[:16], 2 * t)
    np.testing.assert_array_equal(got[16:], 2 * t[::-1])


@pytest.mark.parametrize("fn,k", [(kq.q3k_quantize, 512), (kq.iq4nl_quantize, 64)])
def test_quantizers_zero_and_error(fn, k):
    rng = np.random.default_rng(2)
    deq = kq.q3k_dequantize if fn is kq.q3k_quantize else kq.iq4nl_dequantize
    assert (deq(fn(np.zeros((2, k), np.float32))) == 0).all()
    w = (rng.standard_normal((32, k)) * 0.02).astype(np.float32)
    r = deq(fn(w))
    rel = np.linalg.norm(r - w) / np.linalg.norm(w)
    assert rel < (0.25 if fn is kq.q3k_quantize else 0.12), rel


def test_record_round_trip():
    rng = np.random.default_rng(3)
    g = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    u = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    d = (rng.standard_normal((256, 64)) * 0.02).astype(np.float32)
    rec = kq.pack_q3k_record(g, u, d)
    g2, u2, d2 = kq.unpack_q3k_record(rec, 256, 64)
    np.testing.assert_array_equal(g2, kq.q3k_dequantize(kq.q3k_quantize(g)))
    np.testing.assert_array_equal(d2, kq.iq4nl_dequantize(kq.iq4nl_quantize(d)))
    assert np.linalg.norm(u2 - u) / np.linalg.norm(u) < 0.25

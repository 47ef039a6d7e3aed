"""Pins of the PLE n-gram gather oracle against what the pages and
SplitMix64's published outputs fix ("Edge0-145B: a Qwen MoE with its experts
squeezed, and a 51B table left on the SSD", section "The 51.2B the GPU never
holds"). The hash composition over the n-gram is a reading (parity
unpinned); these tests pin its generator, the table geometry the pages
print, the n-gram structure and the FP8 decode."""

import json
import os

import numpy as np
import pytest

from oracle import ple
from oracle.formats import e4m3_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")


def test_splitmix64_matches_published_outputs():
    g = json.load(open(GOLDEN))
    want = [int(v, 16) for v in g["outputs_hex"]]
    assert ple.splitmix64(g["seed"], len(want)) == want


def test_head_keys_are_the_generator_sequence():
    g = json.load(open(GOLDEN))
    want = [int(v, 16) for v in g["outputs_hex"]]
    assert ple.head_keys()[0] == want


def test_table_geometry_matches_the_pages():
    rows = ple.head_rows()
    assert len(rows) == 16
    assert rows[0] == 20000003                     # "20,000,003 for the first"
    assert sum(rows) == 320001536                  # tensor [160, 320001536]
    assert all(19.9e6 < r < 20.1e6 for r in rows)  # "about 20M rows each"
    assert ple.N_HEADS * ple.ROW_BYTES == 2560     # "sixteen rows of 160 bytes is 2,560 bytes"
    assert sum(rows) * ple.ROW_BYTES == 51200245760  # the 51.2B-parameter table


def _tokens(rng, T):
    return rng.integers(-1, 248000, T + 2).astype(np.int64)


def test_rows_fall_in_their_head():
    rng = np.random.default_rng(1)
    sizes = [101 + 7 * h for h in range(16)]
    off = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    r = ple.ple_rows(_tokens(rng, 50), sizes)
    assert r.shape == (50, 16)
    assert ((r >= off) & (r < off + np.array(sizes))).all()


def test_bigram_heads_ignore_the_oldest_token():
    """Heads 0..7 read (t-1, t), heads 8..15 (t-2, t-1, t): changing the
    token two back moves no 2-gram row and (for large heads) nearly every
    3-gram row."""
    rng = np.random.default_rng(2)
    sizes = ple.head_rows()
    for _ in range(20):
        a = _tokens(rng, 1)
        b = a.copy()
        b[0] = (a[0] + 12345) % 248000
        ra, rb = ple.ple_rows(a, sizes), ple.ple_rows(b, sizes)
        assert np.array_equal(ra[:, :8], rb[:, :8])
        assert (ra[:, 8:] != rb[:, 8:]).sum() >= 6


def test_each_position_sees_its_own_window():
    """Token i's rows depend on tokens i, i+1, i+2 of the array only: the
    rows of a batch are those of its tokens computed one window at a time."""
    rng = np.random.default_rng(3)
    sizes = [997] * 16
    toks = _tokens(rng, 12)
    whole = ple.ple_rows(toks, sizes)
    for i in range(12):
        assert np.array_equal(whole[i], ple.ple_rows(toks[i:i + 3], sizes)[0])


def test_order_of_the_ngram_matters():
    rng = np.random.default_rng(4)
    sizes = ple.head_rows()
    a = _tokens(rng, 1)
    b = a[[0, 2, 1]]
    assert (ple.ple_rows(a, sizes) != ple.ple_rows(b, sizes)).any()


def test_gather_is_the_decoded_rows():
    rng = np.random.default_rng(5)
    sizes = [31 + h for h in range(16)]
    table = rng.integers(0, 256, (sum(sizes), 160), dtype=np.uint8)
    toks = _tokens(rng, 9)
    got = ple.ple_gather(toks, table, sizes)
    rows = ple.ple_rows(toks, sizes)
    for i in range(9):
        for h in range(16):
            np.testing.assert_array_equal(got[i, h], e4m3_decode(table[rows[i, h]]))


def test_empty_batch():
    assert ple.ple_rows(np.array([-1, -1]), [5] * 16).shape == (0, 16)

"""PLE n-gram embedding gather, plain NumPy.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (see the package docstring).

Follows "Edge0-145B: a Qwen MoE with its experts squeezed, and a 51B table
left on the SSD", section "The 51.2B the GPU never holds", and the parts
table of section "The base, byte for byte" (one FP8 tensor [160, 320001536]):
the table is Qwen's n-gram embedding with n-gram size 3, 8 hash heads per
n-gram length, 16 heads of about 20M rows each (the first 20,000,003), rows
of 160 FP8 values; each token hashes its last two and its last three tokens
into 16 rows, 2,560 bytes a token.

Readings (the pages give neither the hash nor the later head sizes):

* heads 0..7 hash the 2-gram (t-1, t), heads 8..15 the 3-gram (t-2, t-1, t);
  a position before the start of the sequence holds the id -1;
* head h's row is mix64(key) mod V_h with key = sum_j (tok_j + 1) K[h][j]
  (mod 2^64) over the n-gram's tokens oldest first, where mix64 is the
  SplitMix64 output function and K[h][j] = mix64((3h + j + 1) * GOLDEN) is
  output 3h + j + 1 of SplitMix64 started from seed 0 (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014);
* head h's rows follow those of heads < h in the table; V_0 = 20,000,003
  and the other 300,001,533 rows are split as evenly as possible over heads
  1..15, the first three taking one row more;
* the FP8 format is E4M3 (OCP E4M3FN, as everywhere else on the pages) with
  no per-row scale; the gathered rows are the decoded values.

The hash composition (the key over the n-gram) is a reading with nothing on
the pages to check it against: parity unpinned beyond SplitMix64's published
outputs and the structural properties in tests/test_oracle_ple.py.
"""

import numpy as np

from .formats import e4m3_decode

N_HEADS = 16
HEADS_PER_NGRAM = 8
ROW_BYTES = 160
TOTAL_ROWS = 320001536
FIRST_HEAD_ROWS = 20000003
GOLDEN = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def mix64(z):
    """SplitMix64's output function on Python ints (exact, mod 2^64)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def splitmix64(seed, n):
    """The first n outputs of SplitMix64 from `seed`: state += GOLDEN, then
    the output function of the state."""
    out, s = [], seed & _M64
    for _ in range(n):
        s = (s + GOLDEN) & _M64
        out.append(mix64(s))
    return out


def head_rows():
    """Rows per head (the reading above); they sum to the table's 320,001,536."""
    rest, n = TOTAL_ROWS - FIRST_HEAD_ROWS, N_HEADS - 1
    base, extra = divmod(rest, n)
    return [FIRST_HEAD_ROWS] + [base + (1 if h <= extra else 0) for h in range(1, N_HEADS)]


def head_keys():
    """K[h][j] = SplitMix64 output 3h + j + 1 from seed 0."""
    seq = splitmix64(0, 3 * N_HEADS)
    return [[seq[3 * h + j] for j in range(3)] for h in range(N_HEADS)]


def ple_rows(tokens, rows_per_head):
    """Global table rows [T][16] for the T tokens of `tokens` (length T + 2:
    the two ids before the batch, then the batch)."""
    toks = [int(v) for v in np.asarray(tokens).ravel()]
    T = len(toks) - 2
    K = head_keys()
    off = np.concatenate([[0], np.cumsum(rows_per_head)[:-1]]).astype(np.int64)
    out = np.zeros((max(T, 0), N_HEADS), dtype=np.int64)
    for i in range(T):
        for h in range(N_HEADS):
            n = 2 if h < HEADS_PER_NGRAM else 3
            gram = toks[i + 3 - n:i + 3]                 # oldest first, ends at token i
            key = 0
            for j, tok in enumerate(gram):
                key = (key + ((tok + 1) & _M64) * K[h][j]) & _M64
            out[i, h] = off[h] + mix64(key) % int(rows_per_head[h])
    return out


def ple_gather(tokens, table, rows_per_head):
    """fp64 [T][16][row_bytes]: the E4M3 values of each token's 16 rows."""
    rows = ple_rows(tokens, rows_per_head)
    table = np.asarray(table, dtype=np.uint8)
    return e4m3_decode(table[rows.ravel()]).reshape(rows.shape[0], N_HEADS, table.shape[1])

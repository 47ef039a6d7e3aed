"""Parity of lmoe_ple_gather (the PLE n-gram embedding gather) with the
oracle, bit for bit: the gathered values are E4M3 codes decoded to bf16,
which is exact, and the rows come from integer hashing."""

import numpy as np
import pytest

from oracle import ple
from oracle.formats import e4m3_decode

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _bits(vals):
    """bf16 bit patterns of exactly representable values (NaN as a mask)."""
    v = np.asarray(vals, dtype=np.float64)
    nan = np.isnan(v)
    # exact in bf16, so the top half of the fp32 pattern (keeps -0)
    b = (np.where(nan, 0.0, v).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return b, nan


def _check(got_bits, want_vals):
    want, nan = _bits(want_vals)
    got = got_bits.view(np.uint16)
    got_nan = (got & 0x7F80) == 0x7F80
    assert np.array_equal(got_nan & ((got & 0x7F) != 0), nan), "NaN positions differ"
    assert np.array_equal(got[~nan], want[~nan])


def _run(tokens, table, sizes, row_bytes):
    from latent_mixture_experts_amd import lmoe
    T = len(tokens) - 2
    tk = torch.from_numpy(np.asarray(tokens, dtype=np.int32)).cuda()
    out = torch.empty(T, 16, row_bytes, dtype=torch.int16, device="cuda")
    lmoe.ple_gather(tk, table, sizes, out, row_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("T,row_bytes", [(37, 160), (1, 160), (5, 32), (64, 1024)])
def test_small_table(T, row_bytes):
    rng = np.random.default_rng(T * 1000 + row_bytes)
    sizes = [101 + 7 * h for h in range(16)]
    table = rng.integers(0, 256, (sum(sizes), row_bytes), dtype=np.uint8)
    toks = rng.integers(-1, 248000, T + 2)
    toks[0] = -1                                   # the sequence starts inside the window
    print("case ple small table T", T, "row_bytes", row_bytes, flush=True)
    got = _run(toks, torch.from_numpy(table).cuda(), sizes, row_bytes)
    _check(got, ple.ple_gather(toks, table, sizes))


def test_all_codes_decode():
    """Every one of the 256 E4M3 codes, in one row of 256 bytes."""
    sizes = [1] * 16
    table = np.tile(np.arange(256, dtype=np.uint8), (16, 1))
    toks = np.array([3, 4, 5])
    got = _run(toks, torch.from_numpy(table).cuda(), sizes, 256)
    _check(got, ple.ple_gather(toks, table, sizes))


def test_empty_batch():
    from latent_mixture_experts_amd import lmoe
    out = torch.empty(0, 16, 160, dtype=torch.int16, device="cuda")
    lmoe.ple_gather(torch.tensor([-1, -1], dtype=torch.int32, device="cuda"),
                    torch.zeros(16, 160, dtype=torch.uint8, device="cuda"), [1] * 16, out)


def test_full_table_sampled():
    """The table at its full size (320,001,536 rows of 160 bytes, 51.2 GB on
    the device, head sizes as read from the pages), 4096 tokens; 48 sampled
    tokens checked against the oracle's rows, read back from the device."""
    sizes = ple.head_rows()
    n = sum(sizes)
    table = torch.empty(n, 160, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    step = 1 << 22
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        table[r0:r1] = torch.randint(0, 256, (r1 - r0, 160), generator=g, device="cuda",
                                     dtype=torch.uint8)
    rng = np.random.default_rng(8)
    T = 4096
    toks = rng.integers(-1, 248000, T + 2)
    print("case ple full table T", T, flush=True)
    got = _run(toks, table, sizes, 160)
    for i in sorted(rng.choice(T, 48, replace=False).tolist()):
        rows = ple.ple_rows(toks[i:i + 3], sizes)[0]
        vals = table[torch.from_numpy(rows).cuda()].cpu().numpy()
        _check(got[i], e4m3_decode(vals))
    del table
    torch.cuda.empty_cache()

"""The library's device packers against the oracle's quantizers: byte work,
so bit-exact."""

import numpy as np
import pytest

import oracle
from oracle import formats as fm

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _lm():
    from latent_mixture_experts_amd import lmoe
    return lmoe


def _masters(shape, seed, std=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * std).astype(np.float32)
    return w


def test_pack_bf16_bit_exact():
    lm = _lm()
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    ties = (np.arange(1, 3000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, [0.0, -0.0]]).astype(np.float32)
    src = torch.from_numpy(v).cuda()
    dst = torch.empty(v.size, dtype=torch.int16, device="cuda")
    lm.pack_bf16(src, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    want = fm.f32_to_bf16_bits(v)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("rows,cols,std", [(64, 256, 0.02), (5, 96, 1.0), (3, 64, 1e-6)])
def test_pack_blocks_bit_exact(bits, rows, cols, std):
    lm = _lm()
    w = _masters((rows, cols), 10 + bits, std)
    w[0, :32] = 0.0                      # an all-zero block
    w[1, 5] = 127.0 / 128.0 * 3          # a tie-prone value
    src = torch.from_numpy(w).cuda()
    dst = torch.empty(lm.du_matrix_bytes(rows, cols, bits), dtype=torch.uint8, device="cuda")
    lm.pack_blocks(src, bits, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), fm.pack_du(w, bits))


@pytest.mark.parametrize("ell,f", [(128, 64), (256, 96)])
def test_pack_expert_records_bit_exact(ell, f):
    lm = _lm()
    n = 3
    rng = np.random.default_rng(20 + ell)
    g = (rng.standard_normal((n, f, ell)) * 0.02).astype(np.float32)
    u = (rng.standard_normal((n, f, ell)) * 0.02).astype(np.float32)
    d = (rng.standard_normal((n, ell, f)) * 0.02).astype(np.float32)
    g[1] = 0.0                            # an all-zero matrix: ts = 1
    u[2, 0, :16] = 0.0                    # an all-zero block
    rec = lm.expert_record_bytes(ell, f)
    dst = torch.empty(n, rec, dtype=torch.uint8, device="cuda")
    lm.pack_expert_records(torch.from_numpy(g).cuda(), torch.from_numpy(u).cuda(),
                           torch.from_numpy(d).cuda(), dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    for e in range(n):
        assert np.array_equal(got[e], fm.pack_expert_record(g[e], u[e], d[e])), "expert %d" % e

"""The C-ABI library loads, exports every symbol include/lmoe.h declares, and
rejects bad arguments on the host (no compute call needs a GPU here)."""

import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmoe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmoe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from latent_mixture_experts_amd import lmoe
    return lmoe.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "lmoe_forward" in names and "lmoe_create" in names and len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_strerror(lib):
    from latent_mixture_experts_amd import lmoe
    for c in (lmoe.OK, lmoe.EINVAL, lmoe.ENOMEM, lmoe.EHIP, lmoe.ESTATE, lmoe.EUNSUPPORTED):
        assert lib.lmoe_strerror(c)
    assert lib.lmoe_strerror(-99) == b"unknown error code"


@pytest.mark.parametrize("ell,f", [(1792, 640), (1280, 640), (128, 64), (64, 32)])
def test_record_bytes_match_oracle(lib, ell, f):
    assert lib.lmoe_expert_record_bytes(ell, f) == oracle.expert_record_bytes(ell, f)


@pytest.mark.parametrize("rows,cols,bits", [(1792, 2560, 8), (2560, 1280, 4), (64, 32, 4)])
def test_du_bytes_match_oracle(lib, rows, cols, bits):
    assert lib.lmoe_du_matrix_bytes(rows, cols, bits) == oracle.du_group_bytes(rows, cols, bits)


def _create(lib, **kw):
    from latent_mixture_experts_amd import lmoe
    base = dict(hidden=256, latent=128, n_experts=16, top_k=2, n_groups=2, expert_ffn=64,
                shared_ffn=64, du_bits=8, max_tokens=4, has_router_bias=0, expert_format=0)
    base.update(kw)
    d = lmoe.Dims(*[base[f] for f, _ in lmoe.Dims._fields_])
    h = ctypes.c_void_p()
    return lib.lmoe_create(ctypes.byref(d), 0, ctypes.byref(h)), h


@pytest.mark.parametrize("kw,code", [
    (dict(du_bits=6), -1), (dict(top_k=17), -1), (dict(hidden=0), -1), (dict(max_tokens=0), -1),
    (dict(has_router_bias=2), -1), (dict(hidden=200), -5), (dict(latent=96), -5),
    (dict(expert_ffn=48), -5), (dict(n_experts=2048), -5), (dict(n_groups=65), -5),
    # 64 groups at T 8: the decode U kernel's partial sums need more LDS than a CU has
    (dict(n_groups=64, max_tokens=8), -5),
])
def test_create_rejects_bad_dims_on_host(lib, kw, code):
    rc, h = _create(lib, **kw)
    assert rc == code and not h.value
    assert lib.lmoe_last_error()


def test_null_arguments(lib):
    assert lib.lmoe_create(None, 0, None) == -1
    assert lib.lmoe_forward(None, None, 1, None, None, None) == -1
    assert lib.lmoe_load_weights(None, None, None) == -1
    lib.lmoe_destroy(None)


def test_ple_gather_argument_checks_on_host(lib):
    """lmoe_ple_gather validates on the host before touching the device:
    bad row widths, negative T, a head without rows and NULL pointers are
    EINVAL; T == 0 is a no-op."""
    from latent_mixture_experts_amd import lmoe
    rows = (ctypes.c_int64 * 16)(*([5] * 16))
    dummy = ctypes.c_void_p(16)                     # never dereferenced on these paths
    f = lib.lmoe_ple_gather
    assert f(dummy, 0, dummy, rows, 160, dummy, None) == lmoe.OK
    assert f(None, 0, None, rows, 160, None, None) == lmoe.OK
    assert f(dummy, -1, dummy, rows, 160, dummy, None) == lmoe.EINVAL
    assert f(dummy, 4, dummy, rows, 100, dummy, None) == lmoe.EINVAL
    assert f(dummy, 4, dummy, rows, 0, dummy, None) == lmoe.EINVAL
    assert f(dummy, 4, dummy, rows, 2048, dummy, None) == lmoe.EINVAL
    assert f(None, 4, dummy, rows, 160, dummy, None) == lmoe.EINVAL
    assert f(dummy, 4, dummy, None, 160, dummy, None) == lmoe.EINVAL
    bad = (ctypes.c_int64 * 16)(*([5] * 15 + [0]))
    assert f(dummy, 4, dummy, bad, 160, dummy, None) == lmoe.EINVAL


def test_q3k_record_sizes_and_refusals(lib):
    """The Q3_K record sizes the pages print, and the shapes lmoe_create
    refuses for Q3_K experts (a latent not a multiple of 256)."""
    from latent_mixture_experts_amd import lmoe
    assert lmoe.expert_record_bytes(1792, 640, 1) == 1630720
    assert lmoe.expert_record_bytes(1280, 640, 1) == 1164800
    assert lmoe.expert_record_bytes(1792, 640, 0) == lmoe.expert_record_bytes(1792, 640)
    assert lmoe.expert_record_bytes(1792, 640, 7) == 0
    for kw, code in ((dict(latent=128), lmoe.EUNSUPPORTED), (dict(expert_format=2), lmoe.EINVAL)):
        a = dict(hidden=256, latent=256, n_experts=16, top_k=2, n_groups=2, expert_ffn=64,
                 shared_ffn=64, du_bits=8, max_tokens=4, has_router_bias=0, expert_format=1)
        a.update(kw)
        d = lmoe.Dims(**a)
        h = ctypes.c_void_p()
        assert lib.lmoe_create(ctypes.byref(d), 0, ctypes.byref(h)) == code, kw

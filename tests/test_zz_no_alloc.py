"""lmoe_forward_noalloc: the decode forward on the static per-GPU scratch
array, through the C ABI, against lmoe_forward on the handle's workspace
(same kernels: bit-identical y) and against the oracle's bar. Two calls in a
row, the second with fewer tokens; then a call on another handle of other
shapes on the same GPU (the array keeps the last call's contents)."""

import numpy as np
import pytest

from cases import Case, assert_close
from latent_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _layer(case, max_tokens=8):
    from latent_mixture_experts_amd import lmoe
    w = case.w
    layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                       w.shared_ffn, w.du_bits, max_tokens, has_router_bias=w.router_bias)
    layer.load(case.blobs)
    return layer


def _both(layer, case, T):
    x = torch.from_numpy(np.ascontiguousarray(case.x[:T])).cuda()
    y_ref = torch.full((T, case.w.hidden), float("nan"), device="cuda")
    y_na = torch.full((T, case.w.hidden), float("nan"), device="cuda")
    layer.forward(x, y_ref)
    layer.forward_noalloc(x, y_na)
    torch.cuda.synchronize()
    return y_ref.cpu().numpy(), y_na.cpu().numpy()


@pytest.mark.parametrize("name", ["145b_decode", "tiny"])
def test_noalloc_matches_forward(name):
    w = wl.WORKLOADS[name]
    c = Case(w, tokens=8)
    layer = _layer(c)
    for T in (4, 2):
        print("case noalloc %s T %d" % (name, T), flush=True)
        ref, got = _both(layer, c, T)
        assert np.array_equal(got, ref), "noalloc y differs from lmoe_forward (T=%d)" % T
        assert_close(got, c.expect(T)["y"], "noalloc y vs oracle (T=%d)" % T)
    layer.close()


def test_noalloc_after_another_handle():
    """A 120B-shaped handle then the tiny one on the same scratch."""
    for name, T in (("120b_decode", 5), ("tiny", 3)):
        c = Case(wl.WORKLOADS[name], tokens=T)
        layer = _layer(c)
        print("case noalloc %s T %d" % (name, T), flush=True)
        ref, got = _both(layer, c, T)
        assert np.array_equal(got, ref)
        layer.close()


def test_noalloc_refusals():
    from latent_mixture_experts_amd import lmoe
    c = Case(wl.WORKLOADS["tiny"], tokens=4)
    layer = _layer(c, max_tokens=16)
    x = torch.zeros(16, 256, device="cuda")
    y = torch.zeros(16, 256, device="cuda")
    with pytest.raises(lmoe.LmoeError) as e:
        layer.forward_noalloc(x, y, T=12)                 # prefill sizes: not served
    assert e.value.code == lmoe.EUNSUPPORTED
    with pytest.raises(lmoe.LmoeError) as e:
        layer.forward_noalloc(x, x, T=2)
    assert e.value.code == lmoe.EINVAL
    with pytest.raises(lmoe.LmoeError) as e:
        layer.forward_noalloc(x, y, T=0)
    assert e.value.code == lmoe.EINVAL
    # a layer whose decode workspace at T 4 exceeds the 16 MiB array (the
    # size is refused before the weights are looked at)
    big = lmoe.Layer(4096, 4096, 64, 8, 64, 256, 4096, 8, 4)
    xb = torch.zeros(4, 4096, device="cuda")
    yb = torch.zeros(4, 4096, device="cuda")
    with pytest.raises(lmoe.LmoeError) as e:
        big.forward_noalloc(xb, yb, T=4)
    assert e.value.code == lmoe.EUNSUPPORTED
    big.close()
    layer.close()

"""Parity of lmoe_forward_block (x += layer(RMSNorm(x))) with the oracle,
layer by layer with teacher forcing: layer l of the oracle reads the GPU's
own fp32 x_l, so rounding upstream cannot legitimately flip a near-tie
downstream. Each layer's update x_{l+1} - x_l is held to the spec bar
and its routed part to 1e-4; the end-to-end drift against the oracle's own
stack is printed, not gated."""

import numpy as np
import pytest

import oracle
from cases import assert_close, dims_of, rel_errors
from latent_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _layer_blobs(w, d, seed, layer, xn):
    m = wl.masters(w, seed, layer)
    lg = oracle.router_logits(xn, oracle.f32_to_bf16_bits(m["router"]), m["router_bias"])
    idx, _ = oracle.select_topk(lg, w.top_k)
    m["expert_ids"] = sorted(set(idx.ravel().tolist()))
    return oracle.pack_layer(d, m)


def run_stack(w, n_layers, T, seed=0, eps=1e-6):
    from latent_mixture_experts_amd import lmoe
    d = dims_of(w)
    x0 = wl.x(w, seed, 0, tokens=T)
    xg = torch.from_numpy(x0).cuda()
    oracle_blobs = []
    for layer_idx in range(n_layers):
        print("stack layer", layer_idx, "T", T, flush=True)
        xin = xg.cpu().numpy().astype(np.float64)
        xn = oracle.rmsnorm(xin, eps)
        blobs = _layer_blobs(w, d, seed, layer_idx, xn)
        oracle_blobs.append(blobs)
        r = oracle.layer_forward(d, blobs, xn, intermediates=True)
        layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                           w.shared_ffn, w.du_bits, T)
        layer.load(blobs)
        layer.forward_block(xg, eps)
        torch.cuda.synchronize()
        layer.close()
        xout = xg.cpu().numpy().astype(np.float64)
        delta = xout - xin
        rel, mx = assert_close(delta, r["y"], "layer %d update" % layer_idx)
        # the routed part, through the fp32 residual add: allow 1e-4 of its
        # norm plus the rounding of x + y to fp32 (half an ulp per element)
        err = np.linalg.norm(delta - r["y_shared"] - r["y_routed"])
        ulp_noise = np.linalg.norm(np.abs(xout) * 2.0 ** -24)
        bound = 1e-4 * np.linalg.norm(r["y_routed"]) + ulp_noise
        print("  update rel L2 %.3g max/rms %.3g; routed-part error %.3g (bound %.3g)" % (
            rel, mx, err, bound), flush=True)
        assert err <= bound
    want = oracle.stack_forward(d, oracle_blobs, x0, eps)
    drift, _ = rel_errors(xg.cpu().numpy(), want)
    print("end-to-end relative drift after %d layers: %.3g" % (n_layers, drift), flush=True)
    return drift


def test_tiny_stack_8_layers():
    w = wl.WORKLOADS["tiny"]
    for T in (4, 3):
        run_stack(w, 8, T)


def test_145b_stack_2_layers():
    w = wl.WORKLOADS["145b_stack"]
    run_stack(w, 2, w.tokens)


def test_block_rejects_bad_eps():
    from latent_mixture_experts_amd import lmoe
    w = wl.WORKLOADS["tiny"]
    layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                       w.shared_ffn, w.du_bits, 4)
    d = dims_of(w)
    layer.load(_layer_blobs(w, d, 0, 0, np.ones((1, w.hidden))))
    x = torch.zeros(4, w.hidden, device="cuda")
    with pytest.raises(lmoe.LmoeError):
        layer.forward_block(x, eps=-1.0)
